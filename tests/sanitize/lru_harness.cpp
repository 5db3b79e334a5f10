// Host harness of the expert cache's residency bookkeeping (csrc/lru.h),
// built with AddressSanitizer and UndefinedBehaviorSanitizer. Random
// sequences of forwards, prefetches and resets are planned by ExpertLru and by
// a reference model kept here as per-slot records (expert, last use, last
// forward, prefetched flag) searched linearly. Every plan, refusal and count
// must agree, and the slot <-> expert tables must stay a bijection.
#include <cstdint>
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <random>
#include <vector>

#include "lru.h"

namespace {

int g_fail = 0;
#define CHECK(cond, ...)                                         \
  do {                                                           \
    if (!(cond)) {                                               \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                         \
      std::fprintf(stderr, "\n");                                \
      if (++g_fail > 20) std::exit(1);                           \
    }                                                            \
  } while (0)

struct Slot {
  int32_t expert = -1;
  int64_t last = 0;  // stamp of the last call that used or filled it
  int64_t fwd = 0;   // stamp of the last forward that used it
  bool pre = false;  // filled by a prefetch, not used by a forward since
};

struct Model {
  int32_t E, S;
  std::vector<Slot> slots;
  int64_t stamp = 0, last_fwd = 0;
  Model(int32_t e, int32_t s) : E(e), S(s), slots((size_t)s) {}

  int32_t find(int32_t e) const {
    for (int32_t s = 0; s < S; ++s)
      if (slots[(size_t)s].expert == e) return s;
    return -1;
  }
  static std::vector<int32_t> distinct(const int32_t* v, size_t n, int32_t E) {
    std::vector<int32_t> out;
    for (size_t i = 0; i < n; ++i) {
      if (v[i] < 0 || v[i] >= E) continue;
      bool dup = false;
      for (int32_t x : out) dup = dup || x == v[i];
      if (!dup) out.push_back(v[i]);
    }
    return out;
  }
  // LRU victim among the slots ok() admits: smallest last use, lower index first
  template <class Ok>
  int32_t victim(Ok ok) const {
    int32_t v = -1;
    for (int32_t s = 0; s < S; ++s)
      if (ok(s) && (v < 0 || slots[(size_t)s].last < slots[(size_t)v].last)) v = s;
    return v;
  }
  bool forward(const int32_t* idx, size_t P, std::vector<k3::SlotCopy>& copies, int64_t& hits,
               int64_t& misses, int64_t& pf_hits) {
    copies.clear();
    hits = misses = pf_hits = 0;
    const int64_t call = ++stamp;
    const std::vector<int32_t> u = distinct(idx, P, E);
    if ((int32_t)u.size() > S) return false;
    for (int32_t e : u) {
      const int32_t s = find(e);
      if (s < 0) continue;
      slots[(size_t)s].last = call;
      ++hits;
      pf_hits += slots[(size_t)s].pre ? 1 : 0;
    }
    for (int32_t e : u) {
      if (find(e) >= 0) continue;
      const int32_t v = victim([&](int32_t s) { return slots[(size_t)s].last < call; });
      if (v < 0) return false;
      slots[(size_t)v].expert = e;
      slots[(size_t)v].last = call;
      copies.push_back({e, v});
      ++misses;
    }
    for (int32_t e : u) {
      Slot& sl = slots[(size_t)find(e)];
      sl.pre = false;
      sl.fwd = call;
    }
    last_fwd = call;
    return true;
  }
  int prefetch(const int32_t* ex, int32_t n, std::vector<k3::SlotCopy>& copies) {
    copies.clear();
    const int64_t pst = ++stamp;
    auto eligible = [&](int32_t s) {
      const Slot& sl = slots[(size_t)s];
      return (last_fwd == 0 || sl.fwd != last_fwd) && sl.last < pst;
    };
    const std::vector<int32_t> u = distinct(ex, (size_t)n, E);
    int32_t need = 0, refresh = 0, free_slots = 0;
    for (int32_t e : u) {
      const int32_t s = find(e);
      if (s < 0)
        ++need;
      else if (eligible(s))
        ++refresh;
    }
    for (int32_t s = 0; s < S; ++s) free_slots += eligible(s) ? 1 : 0;
    if (need > free_slots - refresh) return k3::ExpertLru::kRefused;
    for (int32_t e : u) {
      const int32_t s = find(e);
      if (s >= 0 && eligible(s)) slots[(size_t)s].last = pst;
    }
    for (int32_t e : u) {
      if (find(e) >= 0) continue;
      const int32_t v = victim(eligible);
      if (v < 0) return k3::ExpertLru::kBroken;
      slots[(size_t)v].expert = e;
      slots[(size_t)v].last = pst;
      slots[(size_t)v].pre = true;
      copies.push_back({e, v});
    }
    return k3::ExpertLru::kPlanned;
  }
  void forget() {
    for (Slot& s : slots) {
      s.expert = -1;
      s.last = 0;
      s.pre = false;
    }
  }
};

bool same_copies(const std::vector<k3::SlotCopy>& a, const std::vector<k3::SlotCopy>& b) {
  if (a.size() != b.size()) return false;
  for (size_t i = 0; i < a.size(); ++i)
    if (a[i].expert != b[i].expert || a[i].slot != b[i].slot) return false;
  return true;
}

void check_tables(const k3::ExpertLru& lru, const Model& m, int op) {
  for (int32_t s = 0; s < m.S; ++s) {
    const int32_t e = lru.expert_in(s);
    CHECK(e == m.slots[(size_t)s].expert, "op %d: slot %d holds %d, model %d", op, s, e,
          m.slots[(size_t)s].expert);
    if (e >= 0) CHECK(lru.slot_of(e) == s, "op %d: slot_of(%d) = %d, expected %d", op, e, lru.slot_of(e), s);
  }
  for (int32_t e = 0; e < m.E; ++e) {
    const int32_t s = lru.slot_of(e);
    if (s >= 0) CHECK(lru.expert_in(s) == e, "op %d: expert %d -> slot %d holds %d", op, e, s, lru.expert_in(s));
  }
  CHECK(lru.slot_of(-1) == -1 && lru.slot_of(m.E) == -1, "op %d: out-of-range ids map to a slot", op);
}

void run(uint32_t seed, int32_t E, int32_t S, int32_t k, int ops) {
  std::mt19937 rng(seed);
  k3::ExpertLru lru(E, S);
  Model m(E, S);
  std::vector<k3::SlotCopy> c1, c2;
  std::vector<int32_t> perm((size_t)E);
  for (int32_t i = 0; i < E; ++i) perm[(size_t)i] = i;
  // a skewed popularity so hits, misses and evictions all happen
  auto pick = [&](int32_t bound) {
    std::uniform_real_distribution<double> u(0.0, 1.0);
    return (int32_t)(bound * u(rng) * u(rng));
  };
  for (int op = 0; op < ops; ++op) {
    const int kind = (int)(rng() % 10);
    if (kind < 6) {  // forward of T tokens, k distinct experts each, a few dropped pairs
      const int32_t T = 1 + (int32_t)(rng() % 6);
      std::vector<int32_t> idx;
      for (int32_t t = 0; t < T; ++t) {
        std::vector<int32_t> row;
        while ((int32_t)row.size() < k) {
          const int32_t e = perm[(size_t)pick(E)];
          bool dup = false;
          for (int32_t x : row) dup = dup || x == e;
          if (!dup) row.push_back(e);
        }
        for (int32_t e : row) idx.push_back(rng() % 53 == 0 ? (rng() % 2 ? -1 : E + 3) : e);
      }
      int64_t h1, mi1, p1, h2, mi2, p2;
      const bool ok1 = lru.plan_forward(idx.data(), idx.size(), c1, h1, mi1, p1);
      const bool ok2 = m.forward(idx.data(), idx.size(), c2, h2, mi2, p2);
      CHECK(ok1 == ok2, "op %d: forward accepted %d, model %d", op, ok1, ok2);
      if (ok1 && ok2) {
        CHECK(same_copies(c1, c2), "op %d: forward copies differ (%zu vs %zu)", op, c1.size(), c2.size());
        CHECK(h1 == h2 && mi1 == mi2 && p1 == p2, "op %d: counts %lld/%lld/%lld vs %lld/%lld/%lld", op,
              (long long)h1, (long long)mi1, (long long)p1, (long long)h2, (long long)mi2, (long long)p2);
        std::vector<int32_t> sidx(idx.size());
        lru.rename(idx.data(), idx.size(), sidx.data());
        for (size_t p = 0; p < idx.size(); ++p) {
          const bool in = idx[p] >= 0 && idx[p] < E;
          CHECK(in ? (sidx[p] >= 0 && lru.expert_in(sidx[p]) == idx[p]) : sidx[p] == -1,
                "op %d: pair %zu renamed to %d", op, p, sidx[p]);
        }
      }
    } else if (kind < 9) {  // prefetch: a list with repeats, resident and new experts
      const int32_t n = (int32_t)(rng() % (2 * k + 1));
      std::vector<int32_t> ex((size_t)n);
      for (int32_t i = 0; i < n; ++i) ex[(size_t)i] = perm[(size_t)pick(E)];
      const int r1 = lru.plan_prefetch(ex.data(), n, c1);
      const int r2 = m.prefetch(ex.data(), n, c2);
      CHECK(r1 == r2, "op %d: prefetch plan %d, model %d", op, r1, r2);
      CHECK(r1 != k3::ExpertLru::kBroken, "op %d: prefetch ran out of slots after counting", op);
      if (r1 == k3::ExpertLru::kPlanned && r2 == k3::ExpertLru::kPlanned)
        CHECK(same_copies(c1, c2), "op %d: prefetch copies differ", op);
    } else {
      lru.forget();
      m.forget();
    }
    check_tables(lru, m, op);
    if (op % 997 == 0) std::shuffle(perm.begin(), perm.end(), rng);
  }
}

}  // namespace

int main() {
  // (seed, experts, slots, top-k, operations)
  run(1, 8, 2, 2, 4000);
  run(2, 8, 8, 2, 4000);
  run(3, 64, 8, 8, 6000);
  run(4, 64, 20, 8, 6000);
  run(5, 64, 64, 8, 3000);
  run(6, 896, 64, 16, 3000);
  run(7, 896, 448, 16, 2000);
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("lru harness: all checks passed\n");
  return 0;
}
