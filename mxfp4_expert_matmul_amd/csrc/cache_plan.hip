// Device-side planning and filling of the HBM expert cache, so that a cached
// forward needs no host round trip: the routing stays on the GPU, one
// workgroup plans the call against residency tables in device memory, and a
// fill kernel copies the missing experts straight from pinned host memory
// over PCIe. The replacement rule is the host planner's (lru.h), step for
// step, so both count the same hits, misses and prefetch hits on the same
// calls (the pages' LRU expert cache and its raw versus true resident hits:
// ssnai.com decision guide; xugj520.cn run notes, cache statistics).
#include <climits>

#include "k3_kernels.h"
#include "topk_device.h"

namespace k3 {

namespace {

constexpr int kPlanThreads = 256;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint64_t v2u64 __attribute__((ext_vector_type(2)));

// Items i < n with pred(i), compacted in index order: emit(pos, i) for each;
// returns their count on every thread. wsum: 4 ints of LDS.
template <class Pred, class Emit>
__device__ int compact_in_order(int n, Pred pred, Emit emit, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int base = 0;
  for (int i0 = 0; i0 < n; i0 += kPlanThreads) {
    const int i = i0 + tid;
    const bool f = i < n && pred(i);
    const uint64_t bal = __ballot(f);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
    if (lane == 0) wsum[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    const int tot = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (f) emit(off + below, i);
    base += tot;
    __syncthreads();  // wsum is rewritten by the next round
  }
  return base;
}

// Victim keys: key[s] = (last use << 13) | s for a slot that may take an
// expert, all ones for the others and for the padding entries S .. S8 - 1
// (S8 = S rounded up to 8; S < 2^13 and stamps < 2^50). Eligible keys are
// distinct and order the slots by (last use, slot).
__device__ __forceinline__ int round8(int n) { return (n + 7) & ~7; }
__device__ __forceinline__ uint64_t victim_key(bool eligible, int64_t last_use, int s) {
  return eligible ? (((uint64_t)last_use << 13) | (uint64_t)s) : ~0ull;
}

// Slot s is victim r when r eligible keys are smaller than its key, for
// r < want: the first `want` victims are then exactly the slots the host
// planner's repeated least-recently-used choice takes, in its order. Keys
// are read two per 16-byte load, and a slot stops counting once its rank
// reaches `want`. (The callers guarantee at least `want` eligible slots;
// entries left -1 by inconsistent tables are skipped by the placement.)
__device__ void rank_victims(const uint64_t* key, int S, int want, int32_t* vict) {
  if (want <= 0) return;
  for (int r = threadIdx.x; r < want; r += kPlanThreads) vict[r] = -1;
  __syncthreads();
  const int S8 = round8(S);
  for (int s = threadIdx.x; s < S; s += kPlanThreads) {
    const uint64_t ks = key[s];
    if (ks == ~0ull) continue;
    int r = 0;
    for (int q = 0; q < S8 && r < want; q += 8) {
      const v2u64 a = *reinterpret_cast<const v2u64*>(key + q);
      const v2u64 b = *reinterpret_cast<const v2u64*>(key + q + 2);
      const v2u64 c = *reinterpret_cast<const v2u64*>(key + q + 4);
      const v2u64 d = *reinterpret_cast<const v2u64*>(key + q + 6);
      r += (a.x < ks) + (a.y < ks) + (b.x < ks) + (b.y < ks) + (c.x < ks) + (c.y < ks) +
           (d.x < ks) + (d.y < ks);
    }
    if (r < want) vict[r] = s;
  }
}

// Put expert e in slot v, evicting what v held. Within one plan the slots,
// the incoming experts and the evicted experts are all distinct, so the
// threads' writes never meet.
__device__ __forceinline__ bool place(const CacheTables& tb, int e, int v, int S) {
  if (v < 0 || v >= S) return false;
  const int old = tb.expert_in[v];
  if (old >= 0) tb.slot_of[old] = -1;
  tb.expert_in[v] = e;
  tb.slot_of[e] = v;
  return true;
}

}  // namespace

// One workgroup routes and plans a forward. First each wave selects the top
// k of its tokens' logits [T][E] (the selection and gates of the top-k
// kernel, by the same code: topk_device.h) and writes idx and gate [T][k]
// (and the caller's copies when given). Then it plans over the selection
// (P = T k <= S): the distinct experts in order of first appearance; the
// resident ones are hits and their slots are marked used first; each other
// one takes the least recently used slot the call does not use (ties to the
// lower slot) and is listed for copying; every slot the call uses becomes a
// plain resident one, last used by this forward. Writes the selection
// renamed to slots (dropped pairs -1) and the copy list.
template <int V>  // logits per lane: E <= 64 V
__global__ __launch_bounds__(kPlanThreads) void cache_plan_forward_kernel(
    const float* __restrict__ logits, int T, int k, const float* __restrict__ sel_bias, int E,
    int S, CacheTables tb, int32_t* __restrict__ idx, float* __restrict__ gate,
    int32_t* __restrict__ user_idx, float* __restrict__ user_gate, int32_t* __restrict__ sidx) {
  extern __shared__ __attribute__((aligned(16))) uint8_t plan_lds[];
  const int P = T * k;
  uint64_t* key = reinterpret_cast<uint64_t*>(plan_lds);  // [S8] victim keys
  int64_t* lu = reinterpret_cast<int64_t*>(key + round8(S));  // [S] last use
  int32_t* first = reinterpret_cast<int32_t*>(lu + S);  // [E] first position in the selection
  int32_t* sel = first + E;                              // [P] the selection
  int32_t* uniq = sel + P;                               // [P] distinct experts
  int32_t* missv = uniq + P;                             // [P] those not resident
  int32_t* vict = missv + P;                             // [P] their slots
  __shared__ __attribute__((aligned(16))) uint64_t tk_cand[kPlanThreads / 64][kTopkCand];
  __shared__ uint64_t tk_sel[kPlanThreads / 64][64];
  __shared__ int wsum[4];
  __shared__ int64_t s_call;
  __shared__ int s_hits, s_pfh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the top k of each token (waves work alone: wave-private LDS)
  for (int t = wave; t < T; t += kPlanThreads / 64) {
    const float* row = logits + (size_t)t * E;
    const uint64_t mine = topk_token<V>(row, E, k, tk_cand[wave], tk_sel[wave], sel_bias);
    const float g = sel_bias ? topk_gate_unbiased(mine, k, row) : topk_gate_of(mine, k);
    if (lane < k) {
      const int e = topk_key_index(mine);
      const size_t o = (size_t)t * k + lane;
      idx[o] = e;
      gate[o] = g;
      sel[o] = e;
      if (user_idx) user_idx[o] = e;
      if (user_gate) user_gate[o] = g;
    }
  }
  if (tid == 0) {
    s_call = tb.ctr[kCtrStamp] + 1;
    tb.ctr[kCtrStamp] = s_call;
    s_hits = 0;
    s_pfh = 0;
  }
  for (int s = tid; s < S; s += kPlanThreads) lu[s] = tb.last_use[s];
  for (int e = tid; e < E; e += kPlanThreads) first[e] = INT_MAX;
  __syncthreads();
  const int64_t call = s_call;
  for (int p = tid; p < P; p += kPlanThreads) {
    const int e = sel[p];
    if (e >= 0 && e < E) atomicMin(&first[e], p);
  }
  __syncthreads();
  const int nu = compact_in_order(
      P, [&](int p) { const int e = sel[p]; return e >= 0 && e < E && first[e] == p; },
      [&](int pos, int p) { uniq[pos] = sel[p]; }, wsum);
  // hits: their slots are used by this call before any victim is chosen
  for (int i = tid; i < nu; i += kPlanThreads) {
    const int s = tb.slot_of[uniq[i]];
    if (s >= 0 && s < S) {
      lu[s] = call;
      atomicAdd(&s_hits, 1);
      atomicAdd(&s_pfh, tb.pre[s]);
    }
  }
  __syncthreads();
  const int nm = compact_in_order(
      nu, [&](int i) { return tb.slot_of[uniq[i]] < 0; },
      [&](int pos, int i) { missv[pos] = uniq[i]; }, wsum);
  if (nm > 0) {
    for (int s = tid; s < round8(S); s += kPlanThreads)
      key[s] = victim_key(s < S && lu[s] < call, s < S ? lu[s] : 0, s);
    __syncthreads();
  }
  rank_victims(key, S, nm, vict);
  __syncthreads();
  for (int j = tid; j < nm; j += kPlanThreads) {
    const int v = vict[j], e = missv[j];
    if (place(tb, e, v, S)) lu[v] = call;
    tb.fwd_copies[1 + 2 * j] = e;
    tb.fwd_copies[2 + 2 * j] = v;  // the fill skips v = -1
  }
  __syncthreads();
  for (int i = tid; i < nu; i += kPlanThreads) {
    const int s = tb.slot_of[uniq[i]];
    if (s < 0 || s >= S) continue;
    tb.pre[s] = 0;
    tb.fwd_use[s] = call;
  }
  for (int s = tid; s < S; s += kPlanThreads) tb.last_use[s] = lu[s];
  for (int p = tid; p < P; p += kPlanThreads) {
    const int e = sel[p];
    const int v = (e >= 0 && e < E) ? tb.slot_of[e] : -1;
    sidx[p] = (v >= 0 && v < S) ? v : -1;
  }
  if (tid == 0) {
    tb.fwd_copies[0] = nm;
    tb.ctr[kCtrLastFwd] = call;
    tb.ctr[kCtrCalls] += 1;
    tb.ctr[kCtrHits] += s_hits;
    tb.ctr[kCtrMisses] += nm;
    tb.ctr[kCtrPfHits] += s_pfh;
  }
}

// One workgroup plans a prefetch of experts[0..n) (ids outside [0, E) are
// skipped and counted). Slots it may fill: not used by the last planned
// forward (its kernels may still run) and not taken by this prefetch.
// Listed resident experts in such slots are refreshed (which takes their
// slots); each other listed expert takes the least recently used such slot
// and is listed for copying. Refused (counted, nothing changed but the
// stamp) if too few such slots are left.
__global__ __launch_bounds__(kPlanThreads) void cache_plan_prefetch_kernel(
    const int32_t* __restrict__ experts, int n, int E, int S, CacheTables tb) {
  extern __shared__ __attribute__((aligned(16))) uint8_t plan_lds[];
  uint64_t* key = reinterpret_cast<uint64_t*>(plan_lds);  // [S8] victim keys
  int64_t* lu = reinterpret_cast<int64_t*>(key + round8(S));  // [S]
  int32_t* first = reinterpret_cast<int32_t*>(lu + S);  // [E]
  int32_t* uniq = first + E;                             // [E] distinct listed experts
  int32_t* newv = uniq + E;                              // [E] those not resident
  int32_t* vict = newv + E;                              // [S]
  uint8_t* elig = reinterpret_cast<uint8_t*>(vict + S);  // [S]
  __shared__ int wsum[4];
  __shared__ int64_t s_pst;
  __shared__ int s_ignored, s_refreshed, s_free;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_pst = tb.ctr[kCtrStamp] + 1;
    tb.ctr[kCtrStamp] = s_pst;
    s_ignored = s_refreshed = s_free = 0;
  }
  __syncthreads();
  const int64_t pst = s_pst, last_fwd = tb.ctr[kCtrLastFwd];
  for (int s0 = 0; s0 < S; s0 += kPlanThreads) {
    const int s = s0 + tid;
    bool e = false;
    if (s < S) {
      lu[s] = tb.last_use[s];
      e = (last_fwd == 0 || tb.fwd_use[s] != last_fwd) && lu[s] < pst;
      elig[s] = e ? 1 : 0;
    }
    const uint64_t bal = __ballot(e);
    if ((tid & 63) == 0 && bal) atomicAdd(&s_free, (int)__builtin_popcountll(bal));
  }
  for (int e = tid; e < E; e += kPlanThreads) first[e] = INT_MAX;
  __syncthreads();
  for (int p = tid; p < n; p += kPlanThreads) {
    const int e = experts[p];
    if (e >= 0 && e < E)
      atomicMin(&first[e], p);
    else
      atomicAdd(&s_ignored, 1);
  }
  __syncthreads();
  const int nu = compact_in_order(
      n, [&](int p) { const int e = experts[p]; return e >= 0 && e < E && first[e] == p; },
      [&](int pos, int p) { uniq[pos] = experts[p]; }, wsum);
  const int nn = compact_in_order(
      nu, [&](int i) { return tb.slot_of[uniq[i]] < 0; },
      [&](int pos, int i) { newv[pos] = uniq[i]; }, wsum);
  for (int i = tid; i < nu; i += kPlanThreads) {
    const int s = tb.slot_of[uniq[i]];
    if (s >= 0 && s < S && elig[s]) atomicAdd(&s_refreshed, 1);
  }
  __syncthreads();
  if (nn > s_free - s_refreshed) {
    if (tid == 0) {
      tb.pf_copies[0] = 0;
      tb.ctr[kCtrPfRefused] += 1;
      tb.ctr[kCtrIgnored] += s_ignored;
    }
    return;
  }
  for (int i = tid; i < nu; i += kPlanThreads) {
    const int s = tb.slot_of[uniq[i]];
    if (s >= 0 && s < S && elig[s]) {
      lu[s] = pst;
      elig[s] = 0;
    }
  }
  __syncthreads();
  if (nn > 0) {
    for (int s = tid; s < round8(S); s += kPlanThreads)
      key[s] = victim_key(s < S && elig[s] != 0, s < S ? lu[s] : 0, s);
    __syncthreads();
  }
  rank_victims(key, S, nn, vict);
  __syncthreads();
  for (int j = tid; j < nn; j += kPlanThreads) {
    const int v = vict[j], e = newv[j];
    if (place(tb, e, v, S)) {
      lu[v] = pst;
      tb.pre[v] = 1;
    }
    tb.pf_copies[1 + 2 * j] = e;
    tb.pf_copies[2 + 2 * j] = v;
  }
  __syncthreads();
  for (int s = tid; s < S; s += kPlanThreads) tb.last_use[s] = lu[s];
  if (tid == 0) {
    tb.pf_copies[0] = nn;
    tb.ctr[kCtrPrefetched] += nn;
    tb.ctr[kCtrIgnored] += s_ignored;
  }
}

// Copies the listed experts (count, then (expert, slot) pairs) from host
// memory into their arena slots: work item (copy j, 64 KB chunk c of the
// expert's six tensors, in order); workgroups stride over the items, so the
// grid need not know the count. Entries outside [0, E) x [0, S) are skipped.
__global__ __launch_bounds__(kPlanThreads) void cache_fill_kernel(const int32_t* __restrict__ copies,
                                                                  int max_copies, int E, int S,
                                                                  FillPlan fp) {
  const int n = min(copies[0], max_copies);
  const int nchunk = (int)((fp.total + kFillChunk - 1) / kFillChunk);
  for (int item = blockIdx.x; item < n * nchunk; item += gridDim.x) {
    const int j = item / nchunk, ch = item - j * nchunk;
    const int e = copies[1 + 2 * j], s = copies[2 + 2 * j];
    if (e < 0 || e >= E || s < 0 || s >= S) continue;
    const uint64_t lo = (uint64_t)ch * kFillChunk;
    const uint64_t hi = lo + kFillChunk < fp.total ? lo + kFillChunk : fp.total;
    uint64_t base = 0;
    for (int t = 0; t < kCacheTensors; ++t) {
      const uint64_t b0 = lo > base ? lo : base;
      const uint64_t b1 = hi < base + fp.bytes[t] ? hi : base + fp.bytes[t];
      if (b0 < b1) {
        const v4u* src =
            reinterpret_cast<const v4u*>(fp.src[t] + (uint64_t)e * fp.bytes[t] + (b0 - base));
        v4u* dst = reinterpret_cast<v4u*>(fp.dst[t] + (uint64_t)s * fp.bytes[t] + (b0 - base));
        const int nv = (int)((b1 - b0) >> 4);
        // eight 16-byte loads in flight per thread before their stores
        int i = threadIdx.x;
        for (; i + 7 * kPlanThreads < nv; i += 8 * kPlanThreads) {
          v4u r[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) r[u] = src[i + u * kPlanThreads];
#pragma unroll
          for (int u = 0; u < 8; ++u) dst[i + u * kPlanThreads] = r[u];
        }
        for (; i < nv; i += kPlanThreads) dst[i] = src[i];
      }
      base += fp.bytes[t];
    }
  }
}

// dynamic LDS of the plan kernels (the layouts at the top of each)
size_t cache_plan_forward_lds(int P, int E, int S) {
  return (size_t)((S + 7) & ~7) * 8 + (size_t)S * 8 + (size_t)E * 4 + (size_t)P * 16;
}
size_t cache_plan_prefetch_lds(int E, int S) {
  return (size_t)((S + 7) & ~7) * 8 + (size_t)S * 13 + (size_t)E * 12;
}

// the plan kernel instantiation for E experts: logits per lane V, E <= 64 V
static const void* plan_forward_fn(int E) {
  if (E <= 256) return reinterpret_cast<const void*>(cache_plan_forward_kernel<4>);
  if (E <= 1024) return reinterpret_cast<const void*>(cache_plan_forward_kernel<16>);
  return reinterpret_cast<const void*>(cache_plan_forward_kernel<64>);
}

hipError_t prepare_cache_plan(int P, int E, int S) {
  hipError_t e = hipFuncSetAttribute(plan_forward_fn(E), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)cache_plan_forward_lds(P, E, S));
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(cache_plan_prefetch_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)cache_plan_prefetch_lds(E, S));
}

hipError_t launch_cache_plan_forward(const float* logits, int T, int k, const float* sel_bias,
                                     int E, int S, const CacheTables& tb, int32_t* idx,
                                     float* gate, int32_t* user_idx, float* user_gate,
                                     int32_t* sidx, hipStream_t st) {
  const size_t lds = cache_plan_forward_lds(T * k, E, S);
  if (E <= 256)
    hipLaunchKernelGGL(cache_plan_forward_kernel<4>, dim3(1), dim3(kPlanThreads), lds, st, logits,
                       T, k, sel_bias, E, S, tb, idx, gate, user_idx, user_gate, sidx);
  else if (E <= 1024)
    hipLaunchKernelGGL(cache_plan_forward_kernel<16>, dim3(1), dim3(kPlanThreads), lds, st, logits,
                       T, k, sel_bias, E, S, tb, idx, gate, user_idx, user_gate, sidx);
  else
    hipLaunchKernelGGL(cache_plan_forward_kernel<64>, dim3(1), dim3(kPlanThreads), lds, st, logits,
                       T, k, sel_bias, E, S, tb, idx, gate, user_idx, user_gate, sidx);
  return hipGetLastError();
}

hipError_t launch_cache_plan_prefetch(const int32_t* experts, int n, int E, int S,
                                      const CacheTables& tb, hipStream_t st) {
  hipLaunchKernelGGL(cache_plan_prefetch_kernel, dim3(1), dim3(kPlanThreads),
                     cache_plan_prefetch_lds(E, S), st, experts, n, E, S, tb);
  return hipGetLastError();
}

hipError_t launch_cache_fill(const int32_t* copies, int max_copies, int E, int S,
                             const FillPlan& fp, hipStream_t st) {
  const int64_t nchunk = (int64_t)((fp.total + kFillChunk - 1) / kFillChunk);
  const int64_t items = nchunk * max_copies;
  if (items <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>(items, kFillGrid);
  hipLaunchKernelGGL(cache_fill_kernel, dim3(grid), dim3(kPlanThreads), 0, st, copies, max_copies,
                     E, S, fp);
  return hipGetLastError();
}

}  // namespace k3
