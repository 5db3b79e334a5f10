// Top-k selection and gates of one wave over one token's logits (gfx950),
// shared by the top-k kernel and the decode gate/up GEMV. The order is
// (logit descending, expert index ascending); gates are a softmax over the
// k selected logits (kimi-k3-in-c CHANGELOG walk-through, 0.1.0 section:
// the router picks top-16 of 896; the scoring and normalisation follow the
// plainest reading).
#pragma once
#include "k3_device.h"

namespace k3 {

// One wave per token; the token's logits are read once into registers as
// 64-bit keys that order (value descending, index ascending): the high word
// is the logit's bits mapped to an order-preserving unsigned integer (NaN
// ranks as -inf), the low word the inverted expert index, so equal logits
// rank the lower index higher. Round r takes the largest key strictly below
// the previous round's, so no mask is needed and every step is a compare and
// select (no branches).
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  uint32_t b = __float_as_uint(v);
  if (v != v) b = 0xff800000u;                      // NaN ranks as -inf
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);   // order-preserving map
  return ((uint64_t)b << 32) | (uint32_t)(~(uint32_t)e);
}
__device__ __forceinline__ float topk_key_value(uint64_t key) {
  const uint32_t b = (uint32_t)(key >> 32);
  return __uint_as_float((b & 0x80000000u) ? (b & 0x7fffffffu) : ~b);
}
__device__ __forceinline__ int topk_key_index(uint64_t key) { return (int)~(uint32_t)key; }

// One DPP step of the 64-bit max: combine with the lane selected by CTRL
// (ROW_MASK selects the 16-lane rows that take part; others keep their own).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void max_step(uint64_t& key) {
  const uint32_t lo = (uint32_t)key, hi = (uint32_t)(key >> 32);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROW_MASK, 0xf, false);
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROW_MASK, 0xf, false);
  const uint64_t other = ((uint64_t)ohi << 32) | olo;
  key = other > key ? other : key;
}

// Max over the 64 lanes: quad swaps, half-row and row mirrors give every
// lane its 16-lane row's max; row broadcasts of lanes 15 and 31 carry the
// rows forward so lane 63 holds the wave's max, which every lane then reads.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t key) {
  max_step<0xB1, 0xf>(key);   // quad_perm [1,0,3,2]
  max_step<0x4E, 0xf>(key);   // quad_perm [2,3,0,1]
  max_step<0x141, 0xf>(key);  // row_half_mirror
  max_step<0x140, 0xf>(key);  // row_mirror
  max_step<0x142, 0xa>(key);  // row_bcast15 into rows 1 and 3
  max_step<0x143, 0xc>(key);  // row_bcast31 into rows 2 and 3
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)key, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(key >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Selection (top k keys in descending order) of one wave's V keys per lane.
// The k-th largest of the 64 lane maxima is at most the k-th largest key (k
// distinct keys reach it), and so is tau, its high word with a zero low
// word: every selected key is >= tau.
// Usually few keys pass; they are compacted into LDS and each one's rank
// (the number of passing keys above it) is its position. If more than 64
// pass, k rounds each take the largest key below the previous round's.
// Lane r < k returns selection r. cand: kTopkCand entries, 16-byte aligned
// (the ranking reads up to 7 past the last candidate); sel: 64 entries.
constexpr int kTopkCand = 72;

template <int V>
__device__ uint64_t select_topk(const uint64_t (&key)[V], int k, uint64_t* cand, uint64_t* sel) {
  const int lane = threadIdx.x & 63;
  uint64_t m[V];
#pragma unroll
  for (int j = 0; j < V; ++j) m[j] = key[j];
#pragma unroll
  for (int w = 1; w < V; w *= 2)
#pragma unroll
    for (int j = 0; j + w < V; j += 2 * w) m[j] = m[j + w] > m[j] ? m[j + w] : m[j];
  // tau: the k-th largest high word (the ordered logit bits) of the lane
  // maxima, built bit by bit from the top; a bit stays set when at least k
  // lane maxima reach the prefix with it (a ballot count, no data exchange)
  const uint32_t mh = (uint32_t)(m[0] >> 32);
  uint32_t prefix = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    if (__builtin_popcountll(__ballot(mh >= cand)) >= k) prefix = cand;
  }
  const uint64_t tau = (uint64_t)prefix << 32;
  // compact the keys >= tau (in lane order; their order does not matter)
  int c = 0;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const bool pass = key[j] >= tau;
    const uint64_t bal = __ballot(pass);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
    if (pass && c + below < 64) cand[c + below] = key[j];
    c += __builtin_popcountll(bal);
  }
  if (c <= 64) {
    const uint64_t mine = lane < c ? cand[lane] : 0ull;
    // rank: the passing keys above mine, read eight at a time as LDS
    // broadcasts (every lane reads the same address); entries past c are
    // read but not counted
    int rank = 0;
    for (int i0 = 0; i0 < c; i0 += 8) {
      uint64_t o[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = *reinterpret_cast<const uint4*>(cand + i0 + 2 * q);
        o[2 * q] = ((uint64_t)v.y << 32) | v.x;
        o[2 * q + 1] = ((uint64_t)v.w << 32) | v.z;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) rank += (i0 + q < c && o[q] > mine) ? 1 : 0;
    }
    if (lane < c && rank < k) sel[rank] = mine;
    return lane < k ? sel[lane] : 0ull;
  }
  // many keys above tau: k rounds over all keys
  uint64_t prev = ~0ull, mine = 0ull;
  for (int r = 0; r < k; ++r) {
    uint64_t q[V];
#pragma unroll
    for (int j = 0; j < V; ++j) q[j] = key[j] < prev ? key[j] : 0ull;
#pragma unroll
    for (int w = 1; w < V; w *= 2)
#pragma unroll
      for (int j = 0; j + w < V; j += 2 * w) q[j] = q[j + w] > q[j] ? q[j + w] : q[j];
    const uint64_t best = wave_max_u64(q[0]);
    prev = best;
    if (lane == r) mine = best;
  }
  return mine;
}

// One token row's logits (E of them, V per lane: lane l holds experts
// l + 64 j), and the selection-only bias beside them when there is one.
// Loading is split from selecting so a caller can issue these loads before
// other loads and wait for these alone.
template <int V>
struct TopkRow {
  float l[V], b[V];
};

template <int V>  // logits per lane: E <= 64 * V
__device__ __forceinline__ void topk_load(const float* row, int E, const float* sel_bias,
                                          TopkRow<V>& rw) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int e = lane + 64 * j;
    rw.l[j] = e < E ? row[e] : 0.0f;
    rw.b[j] = (sel_bias && e < E) ? sel_bias[e] : 0.0f;
  }
}

// The top k of a loaded row: lane r < k returns selection r. With the
// selection-only bias the keys rank l[e] + sel_bias[e], added in fp32.
template <int V>
__device__ __forceinline__ uint64_t topk_select(const TopkRow<V>& rw, bool biased, int E, int k,
                                                uint64_t* cand, uint64_t* sel) {
  const int lane = threadIdx.x & 63;
  uint64_t key[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int e = lane + 64 * j;
    const float v = biased ? rw.l[j] + rw.b[j] : rw.l[j];
    key[j] = (e < E) ? topk_key(v, e) : 0ull;  // 0 is below every real key
  }
  return select_topk<V>(key, k, cand, sel);
}

// Keys of token row `row`, then their top k (load and select together).
template <int V>
__device__ __forceinline__ uint64_t topk_token(const float* row, int E, int k, uint64_t* cand,
                                               uint64_t* sel, const float* sel_bias = nullptr) {
  TopkRow<V> rw;
  topk_load<V>(row, E, sel_bias, rw);
  return topk_select<V>(rw, sel_bias != nullptr, E, k, cand, sel);
}

// Gate of lane r < k's selection: exp(l_r - l_0) / sum over the k selected.
__device__ __forceinline__ float topk_gate_of(uint64_t mine, int k) {
  const int lane = threadIdx.x & 63;
  const float v = topk_key_value(mine);
  const float vmax = __shfl(v, 0, 64);
  const float w = (lane < k) ? expf(v - vmax) : 0.0f;
  return w / wave_sum_dpp(w);
}

// Gate of lane r < k's selection under the selection-only bias: the softmax
// of the selected experts' unbiased logits row[e] (NaN counts as -inf) about
// their largest.
__device__ __forceinline__ float topk_gate_unbiased(uint64_t mine, int k, const float* row) {
  const int lane = threadIdx.x & 63;
  float v = -INFINITY;
  if (lane < k) {
    v = row[topk_key_index(mine)];
    if (v != v) v = -INFINITY;
  }
  const float vmax = wave_max(v);
  const float w = (lane < k) ? expf(v - vmax) : 0.0f;
  return w / wave_sum_dpp(w);
}

}  // namespace k3
