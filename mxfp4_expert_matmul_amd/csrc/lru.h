// Residency bookkeeping of the HBM expert cache, with no device calls: which
// arena slot holds which expert, least-recently-used replacement, and the
// raw / true-resident hit accounting the pages distinguish (ssnai.com
// decision guide; xugj520.cn run notes, cache statistics: a hit on an
// expert the prefetcher has just read in is raw, not truly resident).
// cache.cpp performs the copies and kernel launches this plans; the host
// harness under the sanitizers drives it directly.
#pragma once
#include <cstddef>
#include <cstdint>
#include <vector>

namespace k3 {

// One expert to copy into one slot.
struct SlotCopy {
  int32_t expert, slot;
};

class ExpertLru {
 public:
  ExpertLru() = default;
  ExpertLru(int32_t n_experts, int32_t n_slots) { reset(n_experts, n_slots); }

  void reset(int32_t n_experts, int32_t n_slots) {
    E_ = n_experts;
    S_ = n_slots;
    slot_of_.assign((size_t)n_experts, -1);
    expert_in_.assign((size_t)n_slots, -1);
    last_use_.assign((size_t)n_slots, 0);
    seen_.assign((size_t)n_experts, 0);
    fwd_use_.assign((size_t)n_slots, 0);
    pre_.assign((size_t)n_slots, 0);
    uniq_.clear();
    uniq_.reserve((size_t)n_slots);
    stamp_ = last_fwd_ = 0;
  }

  int32_t n_experts() const { return E_; }
  int32_t n_slots() const { return S_; }
  int32_t slot_of(int32_t e) const { return (e >= 0 && e < E_) ? slot_of_[(size_t)e] : -1; }
  int32_t expert_in(int32_t s) const { return expert_in_[(size_t)s]; }

  // Forget every resident expert (after a failed call the arena's contents
  // are not known). Stamps keep counting.
  void forget() {
    for (auto& v : slot_of_) v = -1;
    for (auto& v : expert_in_) v = -1;
    for (auto& v : last_use_) v = 0;
    for (auto& v : pre_) v = 0;
  }

  // Plans a forward over the selection idx[0..P) (entries outside [0, E) are
  // dropped pairs). Returns false, with nothing changed, if the call routes to
  // more distinct experts than there are slots. Otherwise: the call's
  // resident experts are hits (their slots marked used first, so none is
  // evicted for another expert of the call), each other expert takes the
  // least recently used slot this call does not use (ties to the lower slot)
  // and is appended to `copies`; every slot the call uses becomes a plain
  // resident one, off limits to prefetches until a later forward. hits,
  // misses and prefetch_hits (hits on experts a prefetch brought in that no
  // call had used since) are the call's counts.
  bool plan_forward(const int32_t* idx, size_t P, std::vector<SlotCopy>& copies, int64_t& hits,
                    int64_t& misses, int64_t& prefetch_hits) {
    copies.clear();
    hits = misses = prefetch_hits = 0;
    const int64_t call = ++stamp_;
    uniq_.clear();
    for (size_t p = 0; p < P; ++p) {
      const int32_t e = idx[p];
      if (e < 0 || e >= E_ || seen_[(size_t)e] == call) continue;
      seen_[(size_t)e] = call;
      if ((int32_t)uniq_.size() == S_) return false;
      uniq_.push_back(e);
    }
    for (int32_t e : uniq_) {
      const int32_t s = slot_of_[(size_t)e];
      if (s >= 0) {
        last_use_[(size_t)s] = call;
        ++hits;
        prefetch_hits += pre_[(size_t)s];
      }
    }
    for (int32_t e : uniq_) {
      if (slot_of_[(size_t)e] >= 0) continue;
      int32_t v = -1;
      for (int32_t s = 0; s < S_; ++s)
        if (last_use_[(size_t)s] < call && (v < 0 || last_use_[(size_t)s] < last_use_[(size_t)v]))
          v = s;
      // a victim exists: this call uses fewer distinct experts than slots
      place(e, v);
      last_use_[(size_t)v] = call;
      copies.push_back({e, v});
      ++misses;
    }
    for (int32_t e : uniq_) {
      const int32_t s = slot_of_[(size_t)e];
      pre_[(size_t)s] = 0;
      fwd_use_[(size_t)s] = call;
    }
    last_fwd_ = call;
    return true;
  }

  // The selection renamed to slots (dropped pairs become -1).
  void rename(const int32_t* idx, size_t P, int32_t* sidx) const {
    for (size_t p = 0; p < P; ++p) sidx[p] = slot_of(idx[p]);
  }

  // Plans a prefetch of experts[0..n) (ids already checked to lie in
  // [0, E)). Slots it may fill: not used by the last forward (its kernels
  // may still run) and not already taken by this prefetch. Listed resident
  // experts in such slots are refreshed (which takes their slots); the
  // others need a slot each, the least recently used eligible one. Returns
  // kPlanned, or kRefused with nothing changed if too few eligible slots are
  // left (kBroken: a slot ran out after the count, which the count rules
  // out; the tables are then inconsistent and must be forgotten).
  enum PrefetchPlan { kPlanned, kRefused, kBroken };
  PrefetchPlan plan_prefetch(const int32_t* experts, int32_t n, std::vector<SlotCopy>& copies) {
    copies.clear();
    const int64_t pst = ++stamp_;
    auto eligible = [&](int32_t s) {
      return (last_fwd_ == 0 || fwd_use_[(size_t)s] != last_fwd_) && last_use_[(size_t)s] < pst;
    };
    uniq_.clear();
    int32_t refreshed = 0;
    for (int32_t i = 0; i < n; ++i) {
      const int32_t e = experts[i];
      if (seen_[(size_t)e] == pst) continue;
      seen_[(size_t)e] = pst;
      const int32_t s = slot_of_[(size_t)e];
      if (s < 0)
        uniq_.push_back(e);
      else if (eligible(s))
        ++refreshed;
    }
    int32_t free_slots = 0;
    for (int32_t s = 0; s < S_; ++s) free_slots += eligible(s) ? 1 : 0;
    if ((int32_t)uniq_.size() > free_slots - refreshed) return kRefused;
    for (int32_t i = 0; i < n; ++i) {
      const int32_t s = slot_of_[(size_t)experts[i]];
      if (s >= 0 && eligible(s)) last_use_[(size_t)s] = pst;
    }
    for (int32_t e : uniq_) {
      int32_t v = -1;
      for (int32_t s = 0; s < S_; ++s)
        if (eligible(s) && (v < 0 || last_use_[(size_t)s] < last_use_[(size_t)v])) v = s;
      if (v < 0) return kBroken;  // cannot happen after the count above
      place(e, v);
      last_use_[(size_t)v] = pst;
      pre_[(size_t)v] = 1;
      copies.push_back({e, v});
    }
    return kPlanned;
  }

 private:
  // Put expert e in slot v (evicting what v held).
  void place(int32_t e, int32_t v) {
    const int32_t old = expert_in_[(size_t)v];
    if (old >= 0) slot_of_[(size_t)old] = -1;
    expert_in_[(size_t)v] = e;
    slot_of_[(size_t)e] = v;
  }

  int32_t E_ = 0, S_ = 0;
  std::vector<int32_t> slot_of_;    // [E]: slot holding expert e, or -1
  std::vector<int32_t> expert_in_;  // [S]: expert in slot s, or -1
  std::vector<int64_t> last_use_;   // [S]: stamp of the last call that used slot s (0: never)
  std::vector<int64_t> seen_;       // [E]: stamp of the last call that listed expert e
  std::vector<int64_t> fwd_use_;    // [S]: stamp of the last forward that used slot s
  std::vector<uint8_t> pre_;        // [S]: brought in by a prefetch, not used since
  std::vector<int32_t> uniq_;       // scratch: distinct experts of a call
  int64_t stamp_ = 0;               // counts every forward past the routing and every prefetch
  int64_t last_fwd_ = 0;            // stamp of the last planned forward (0: none)
};

}  // namespace k3
