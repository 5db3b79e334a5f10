// Token-to-expert grouping (the chunk-union step of the kimi-k3-in-c
// CHANGELOG walk-through, Unreleased section: within a chunk each routed
// expert is fetched once for all the tokens that picked it).
// The (token, slot) pairs p = t*k + j are bucketed by expert with a stable
// counting sort done in four passes:
//   1. per-block expert histogram (blocks of kGroupChunk pairs),
//   2. per-expert column prefix over the blocks (16 experts x 16 block
//      segments per workgroup): each block's base within each expert, and
//      the expert counts,
//   3. one workgroup: the exclusive prefix sum over experts and the prefill
//      tile list (expert, first row),
//   4. per block, each pair's rank among the block's earlier pairs of the
//      same expert (direct comparison in LDS) gives its slot, so equal
//      experts keep pair order.
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

// Column prefix over blocks for 16 experts per workgroup: thread (c, q)
// handles column e0 + c over segment q of the blocks (16 segments).
// bhist[b][e] becomes the count of expert e in blocks before b; counts[e] its
// total. grid: ceil(E / 16), block 256.
__global__ __launch_bounds__(256) void group_colscan_kernel(int32_t* __restrict__ bhist, int NB,
                                                            int E, int32_t* __restrict__ counts) {
  __shared__ int32_t part[16][16];
  const int c = threadIdx.x & 15, q = threadIdx.x >> 4;
  const int e = blockIdx.x * 16 + c;
  const int per = (NB + 15) / 16;
  const int b0 = q * per, b1 = min(NB, b0 + per);
  int sum = 0;
  if (e < E)
    for (int b = b0; b < b1; ++b) sum += bhist[(size_t)b * E + e];
  part[q][c] = sum;
  __syncthreads();
  int run = 0;
  for (int i = 0; i < q; ++i) run += part[i][c];
  if (e < E) {
    for (int b = b0; b < b1; ++b) {
      const int v = bhist[(size_t)b * E + e];
      bhist[(size_t)b * E + e] = run;
      run += v;
    }
    if (q == 15) counts[e] = run;
  }
}

// Exclusive prefix over experts (each of 1024 threads owns a contiguous run
// of experts), offsets[E] = number of pairs kept, and the tile list.
__global__ __launch_bounds__(1024) void group_scan_kernel(const int32_t* __restrict__ counts, int E,
                                                          int tile_m,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ tiles,
                                                          int32_t* __restrict__ ntiles) {
  __shared__ int32_t part[1024];
  __shared__ int32_t tpart[1024];
  const int tid = threadIdx.x;
  const int per = (E + 1023) / 1024;
  const int lo = tid * per, hi = min(lo + per, E);
  int s = 0, ts = 0;
  for (int e = lo; e < hi; ++e) {
    const int cn = counts[e];
    s += cn;
    ts += (cn + tile_m - 1) / tile_m;
  }
  part[tid] = s;
  tpart[tid] = ts;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 partials
  for (int off = 1; off < 1024; off <<= 1) {
    const int a = (tid >= off) ? part[tid - off] : 0;
    const int b = (tid >= off) ? tpart[tid - off] : 0;
    __syncthreads();
    part[tid] += a;
    tpart[tid] += b;
    __syncthreads();
  }
  int base = part[tid] - s, tbase = tpart[tid] - ts;
  for (int e = lo; e < hi; ++e) {
    const int cn = counts[e];
    const int tl = (cn + tile_m - 1) / tile_m;
    offsets[e] = base;
    for (int i = 0; i < tl; ++i) {
      tiles[2 * (tbase + i)] = e;
      tiles[2 * (tbase + i) + 1] = i * tile_m;
    }
    base += cn;
    tbase += tl;
  }
  if (tid == 1023) {
    offsets[E] = part[1023];
    ntiles[0] = tpart[1023];
  }
}

// Pair p of block b goes to offsets[e] + (pairs of expert e in earlier
// blocks) + (pairs of expert e earlier in this block).
// grid: NB, block kGroupChunk (= 256).
__global__ __launch_bounds__(kGroupChunk) void group_scatter_kernel(
    const int32_t* __restrict__ idx, int P, int E, const int32_t* __restrict__ bhist,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ perm) {
  __shared__ __attribute__((aligned(16))) int32_t ex[kGroupChunk];
  const int tid = threadIdx.x;
  const int p = blockIdx.x * kGroupChunk + tid;
  int e = (p < P) ? idx[p] : -1;
  if (e < 0 || e >= E) e = -1;
  ex[tid] = e;
  __syncthreads();
  if (e < 0) return;
  int rank = 0;
  const int4* ex4 = reinterpret_cast<const int4*>(ex);
  for (int i = 0; i < (tid >> 2); ++i) {
    const int4 v = ex4[i];
    rank += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
  }
  for (int i = tid & ~3; i < tid; ++i) rank += (ex[i] == e);
  perm[offsets[e] + bhist[(size_t)blockIdx.x * E + e] + rank] = p;
}

hipError_t launch_group(const int32_t* idx, int T, const Shape& s, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* bhist, int32_t* tiles,
                        int32_t* ntiles, hipStream_t st) {
  const int P = T * s.k;
  const int NB = (P + kGroupChunk - 1) / kGroupChunk;
  if (NB > 0)
    hipLaunchKernelGGL(group_hist_kernel, dim3(NB), dim3(256), 0, st, idx, P, s.E, bhist);
  // with no pairs the column pass writes zero counts (the scan zero offsets)
  hipLaunchKernelGGL(group_colscan_kernel, dim3((s.E + 15) / 16), dim3(256), 0, st, bhist, NB, s.E,
                     counts);
  hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(1024), 0, st, counts, s.E, kTileM, offsets,
                     tiles, ntiles);
  if (NB > 0)
    hipLaunchKernelGGL(group_scatter_kernel, dim3(NB), dim3(kGroupChunk), 0, st, idx, P, s.E,
                       bhist, offsets, perm);
  return hipGetLastError();
}

}  // namespace k3
