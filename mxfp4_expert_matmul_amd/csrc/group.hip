// Token-to-expert grouping (the chunk-union step of the kimi-k3-in-c
// CHANGELOG walk-through, Unreleased section: within a chunk each routed
// expert is fetched once for all the tokens that picked it).
// The (token, slot) pairs p = t*k + j are bucketed by expert with a stable
// counting sort done in three passes:
//   1. per-block expert histogram (blocks of kGroupChunk pairs),
//   2. one workgroup turns the block histograms into per-block bases
//      (column prefix over blocks), expert counts, the exclusive prefix sum
//      over experts, and the prefill tile list (expert, first row),
//   3. one wave per block places its pairs in order with a wave-level match
//      loop (ballot over equal experts), so equal experts keep pair order.
// Pairs whose expert is outside [0, E) are dropped (they contribute zero).
#include "k3_device.h"
#include "k3_kernels.h"

namespace k3 {

constexpr int kMaxE = 4096;

__global__ __launch_bounds__(256) void group_hist_kernel(const int32_t* __restrict__ idx, int P,
                                                         int E, int32_t* __restrict__ bhist) {
  __shared__ int32_t h[kMaxE];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int p = blockIdx.x * kGroupChunk + threadIdx.x;
  if (p < P) {
    int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  int32_t* out = bhist + (size_t)blockIdx.x * E;
  for (int e = threadIdx.x; e < E; e += 256) out[e] = h[e];
}

__global__ __launch_bounds__(1024) void group_scan_kernel(int32_t* __restrict__ bhist, int NB,
                                                          int E, int tile_m,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ tiles,
                                                          int32_t* __restrict__ ntiles) {
  __shared__ int32_t cnt[kMaxE];
  __shared__ int32_t tl[kMaxE];
  __shared__ int32_t part[1024];
  __shared__ int32_t tpart[1024];
  const int tid = threadIdx.x;
  // 1) column prefix over blocks: bhist[b][e] becomes the count of expert e
  //    in blocks before b.
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int b = 0; b < NB; ++b) {
      int v = bhist[(size_t)b * E + e];
      bhist[(size_t)b * E + e] = run;
      run += v;
    }
    cnt[e] = run;
    tl[e] = (run + tile_m - 1) / tile_m;
  }
  __syncthreads();
  // 2) exclusive prefix over experts: each thread owns a contiguous run.
  const int per = (E + 1023) / 1024;
  const int lo = tid * per, hi = min(lo + per, E);
  int s = 0, ts = 0;
  for (int e = lo; e < hi; ++e) { s += cnt[e]; ts += tl[e]; }
  part[tid] = s;
  tpart[tid] = ts;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 partials
  for (int off = 1; off < 1024; off <<= 1) {
    int a = (tid >= off) ? part[tid - off] : 0;
    int b = (tid >= off) ? tpart[tid - off] : 0;
    __syncthreads();
    part[tid] += a;
    tpart[tid] += b;
    __syncthreads();
  }
  int base = part[tid] - s, tbase = tpart[tid] - ts;
  for (int e = lo; e < hi; ++e) {
    counts[e] = cnt[e];
    offsets[e] = base;
    for (int i = 0; i < tl[e]; ++i) {
      tiles[2 * (tbase + i)] = e;
      tiles[2 * (tbase + i) + 1] = i * tile_m;
    }
    base += cnt[e];
    tbase += tl[e];
  }
  if (tid == 1023) {
    offsets[E] = part[1023];
    ntiles[0] = tpart[1023];
  }
}

__global__ __launch_bounds__(64) void group_scatter_kernel(const int32_t* __restrict__ idx, int P,
                                                           int E,
                                                           const int32_t* __restrict__ bhist,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm) {
  __shared__ int32_t base[kMaxE];
  const int lane = threadIdx.x;
  const int32_t* bh = bhist + (size_t)blockIdx.x * E;
  for (int e = lane; e < E; e += 64) base[e] = offsets[e] + bh[e];
  __syncthreads();
  const int p0 = blockIdx.x * kGroupChunk;
  for (int sub = 0; sub < kGroupChunk; sub += 64) {
    const int p = p0 + sub + lane;
    int e = (p < P) ? idx[p] : -1;
    bool active = (e >= 0 && e < E);
    uint64_t remaining = __ballot(active);
    while (remaining) {
      const int leader = __ffsll((unsigned long long)remaining) - 1;
      const int le = __shfl(e, leader, 64);
      const bool mine = active && (e == le);
      const uint64_t m = __ballot(mine);
      const int b = base[le];
      if (mine) {
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        perm[b + __popcll(m & lt)] = p;
      }
      __syncthreads();  // all lanes read base[le] before it advances
      if (lane == leader) base[le] = b + __popcll(m);
      __syncthreads();
      remaining &= ~m;
    }
  }
}

hipError_t launch_group(const int32_t* idx, int T, const Shape& s, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* bhist, int32_t* tiles,
                        int32_t* ntiles, hipStream_t st) {
  const int P = T * s.k;
  const int NB = (P + kGroupChunk - 1) / kGroupChunk;
  if (NB > 0)
    hipLaunchKernelGGL(group_hist_kernel, dim3(NB), dim3(256), 0, st, idx, P, s.E, bhist);
  // with no pairs the scan alone writes zero counts and offsets
  hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(1024), 0, st, bhist, NB, s.E, kTileM, counts,
                     offsets, tiles, ntiles);
  if (NB > 0)
    hipLaunchKernelGGL(group_scatter_kernel, dim3(NB), dim3(64), 0, st, idx, P, s.E, bhist, offsets,
                       perm);
  return hipGetLastError();
}

}  // namespace k3
