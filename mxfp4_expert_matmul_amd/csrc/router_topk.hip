// Router: fp32 logits l[t,e] = sum_i x[t,i] * Wr[e,i] (+ bias[e]), then per
// token the top-k experts by (logit descending, index ascending) and gates
// renormalised over the selection, gate_j = exp(l_j - l_max) / sum_S exp(.).
// (kimi-k3-in-c CHANGELOG walk-through, 0.1.0 section: the MoE router picks
// top-16 of 896 routed experts; scoring and normalisation are not given on
// the pages and follow the plainest reading.)
#include "k3_device.h"
#include "k3_kernels.h"
#include "topk_device.h"

#include <algorithm>

namespace k3 {

// ---------------------------------------------------------------- logits, small T
// One workgroup (4 waves) per expert row: every thread loads its share of the
// row (d/256 floats, all loads issued before use) and applies it to every
// token of the call; partial sums meet in LDS. HBM-bound: E*d*4 bytes.
template <int TMAX>
__global__ __launch_bounds__(256) void router_gemv_kernel(const uint16_t* __restrict__ x, int T,
                                                          int d, const float* __restrict__ wr,
                                                          const float* __restrict__ bias, int E,
                                                          float* __restrict__ logits) {
  __shared__ float part[4][TMAX];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x;
  const float4* row = reinterpret_cast<const float4*>(wr + (size_t)e * d);
  constexpr int kMaxPer = 8;  // float4 per thread for d <= 8192
  const int n4 = d >> 2;
  // every load is issued, with its index clamped into the row, before any
  // is used (a load behind a branch made the compiler wait for each x load
  // in turn); an out-of-row piece's sum is then dropped by a select
  float4 w[kMaxPer];
  uint2 xv[kMaxPer][TMAX];
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const int i = min(tid + 256 * j, n4 - 1);
    w[j] = row[i];
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
      xv[j][t] = *reinterpret_cast<const uint2*>(x + (size_t)min(t, T - 1) * d + 4 * i);
  }
  float acc[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) acc[t] = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const bool in = tid + 256 * j < n4;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      const uint2 v = xv[j][t];
      float a = acc[t];
      a = fmaf(bf16_bits_to_f32(v.x & 0xffffu), w[j].x, a);
      a = fmaf(bf16_bits_to_f32(v.x >> 16), w[j].y, a);
      a = fmaf(bf16_bits_to_f32(v.y & 0xffffu), w[j].z, a);
      a = fmaf(bf16_bits_to_f32(v.y >> 16), w[j].w, a);
      acc[t] = in ? a : acc[t];  // the same sum, in the same order, as before
    }
  }
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if (t < T) {
      const float s = wave_sum_dpp(acc[t]);
      if (lane == 0) part[wave][t] = s;
    }
  }
  __syncthreads();
  if (tid < T) {
    const float s = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
    logits[(size_t)tid * E + e] = s + (bias ? bias[e] : 0.0f);
  }
}

// ---------------------------------------------------------------- logits, large T
// The fp32 router weights are split once (at handle creation) into three bf16
// terms w = hi + mid + lo, which is exact (24 significant bits = 3 x 8). x is
// bf16, so every product x * term is exact in fp32 and the logits come from
// bf16 MFMAs (v_mfma_f32_16x16x32_bf16) accumulating in fp32: the same
// arithmetic class as an fp32 dot product, at MFMA rate.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ wr, size_t n,
                                                           uint16_t* __restrict__ w3) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const float w = wr[i];
    const uint16_t hi = f32_to_bf16_rne(w);
    const float r1 = w - bf16_bits_to_f32(hi);
    const uint16_t mid = f32_to_bf16_rne(r1);
    const float r2 = r1 - bf16_bits_to_f32(mid);
    w3[i] = hi;
    w3[n + i] = mid;
    w3[2 * n + i] = f32_to_bf16_rne(r2);
  }
}

// Large T: a GEMM of the 3 weight terms [E][d] by x [T][d] on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16). Workgroup tile: 128 experts x 128 tokens; its
// 8 waves are 2 x 4, each 64 experts x 32 tokens (4 x 2 MFMA tiles), and
// each issues half as many copies as with 4 waves per workgroup (the copies
// bound this kernel, and each wave keeps only so many in flight). K is
// walked 32 columns at a time through a ring of 4 LDS stages, copies issued
// 3 steps ahead. Each MFMA operand (16 rows x 32 columns) is copied straight
// into LDS in operand order (lane l's 16 bytes = row l % 16, columns
// 8 (l / 16) .. +7), so its read is one conflict-free ds_read_b128. The
// copies are bounds-checked buffer loads (rows past E or T read zeros).
// MFMA operand lane l: row/column l % 16, 8 consecutive K at 8 (l / 16); both
// operands use the same layout, so any consistent K order is a valid sum.
constexpr int kRtStages = 4;
struct RouterStage {
  uint8_t a[3][8][1024];  // weight terms: 3 x 8 row tiles of 16 experts
  uint8_t b[8][1024];     // x: 8 column tiles of 16 tokens
};

__device__ __forceinline__ void router_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// grid: (ceil(E / 128), ceil(T / 128)), block 512: 8 waves, 2 x 4, each 64
// experts x 32 tokens; copies split 4 per wave (waves 0-5: weight term
// w / 2, row tiles 4 (w % 2) .. +3; waves 6-7: x tiles 4 (w - 6) .. +3).
__global__ __launch_bounds__(512, 1) void router_mfma_kernel(const uint16_t* __restrict__ x, int T,
                                                             int d, const uint16_t* __restrict__ w3,
                                                             const float* __restrict__ bias, int E,
                                                             float* __restrict__ logits) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  __shared__ __attribute__((aligned(16))) RouterStage st0, st1, st2, st3;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * 128, t0 = blockIdx.y * 128;
  const int wm = wave >> 2, wn = wave & 3;
  const int nk = d >> 5;
  const size_t plane = (size_t)E * d;
  const bool wcopy = wave < 6;
  const int term = wave >> 1, rt0 = 4 * (wave & 1), xt0 = 4 * (wave - 6);
  const __amdgpu_buffer_rsrc_t rs = wcopy
      ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(w3 + term * plane), 0,
                                          (int)(plane * 2), 0x00020000)
      : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, (int)((size_t)T * d * 2),
                                          0x00020000);
  const int row0 = wcopy ? e0 + 16 * rt0 : t0 + 16 * xt0;
  const uint32_t voff = (uint32_t)(row0 + r) * (uint32_t)d * 2u + 16u * (uint32_t)g;
  auto issue = [&](RouterStage& S, int ks) __attribute__((always_inline)) {
    const int kb = 64 * min(ks, nk - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint8_t* dst = wcopy ? &S.a[term][rt0 + i][0] : &S.b[xt0 + i][0];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)dst, 16,
                                               (int)(voff + (uint32_t)i * 16u * (uint32_t)d * 2u),
                                               kb, 0, 0);
    }
  };
  v4f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const RouterStage& S) __attribute__((always_inline)) {
    v8bf b[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const v8bf*>(&S.b[2 * wn + j][16 * lane]);
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v8bf a = *reinterpret_cast<const v8bf*>(&S.a[q][4 * wm + i][16 * lane]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[i][j], 0, 0, 0);
      }
  };
  auto step = [&](const RouterStage& Sc, RouterStage& Sn, int s) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt((8 & 15) | ((8 >> 4) << 14) | (7 << 4) | (15 << 8));  // vmcnt(8)
    router_barrier();
    issue(Sn, s + 3);
    compute(Sc);
  };
  issue(st0, 0);
  issue(st1, 1);
  issue(st2, 2);
  for (int s = 0; s < nk; s += 4) {
    step(st0, st3, s);
    if (s + 1 >= nk) break;
    step(st1, st0, s + 1);
    if (s + 2 >= nk) break;
    step(st2, st1, s + 2);
    if (s + 3 >= nk) break;
    step(st3, st2, s + 3);
  }
  __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));
  // result element q of lane l: expert 64 wm + 16 i + 4 g + q, token 32 wn + 16 j + r
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = t0 + 32 * wn + 16 * j + r;
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = e0 + 64 * wm + 16 * i + 4 * g + q;
        if (e < E) logits[(size_t)t * E + e] = acc[i][j][q] + (bias ? bias[e] : 0.0f);
      }
  }
}

hipError_t launch_router_split(const float* wr, int E, int d, uint16_t* w3, hipStream_t st) {
  const size_t n = (size_t)E * d;
  hipLaunchKernelGGL(router_split_kernel, dim3((unsigned)std::min<size_t>((n + 255) / 256, 8192)),
                     dim3(256), 0, st, wr, n, w3);
  return hipGetLastError();
}

hipError_t launch_router_logits(const uint16_t* x, int T, const Shape& s, const float* wr,
                                const uint16_t* wr3, const float* bias, float* logits,
                                hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (T <= kRouterGemvMaxT) {
    dim3 grid(s.E);
    if (T == 1)
      hipLaunchKernelGGL(router_gemv_kernel<1>, grid, dim3(256), 0, st, x, T, s.d, wr, bias, s.E, logits);
    else if (T <= 4)
      hipLaunchKernelGGL(router_gemv_kernel<4>, grid, dim3(256), 0, st, x, T, s.d, wr, bias, s.E, logits);
    else
      hipLaunchKernelGGL(router_gemv_kernel<8>, grid, dim3(256), 0, st, x, T, s.d, wr, bias, s.E, logits);
  } else {
    dim3 grid((s.E + 127) / 128, (T + 127) / 128);
    hipLaunchKernelGGL(router_mfma_kernel, grid, dim3(512), 0, st, x, T, s.d, wr3, bias, s.E, logits);
  }
  return hipGetLastError();
}

template <int V>  // logits per lane: E <= 64 * V
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, const float* __restrict__ sel_bias,
                                                   int32_t* __restrict__ idx,
                                                   float* __restrict__ gate) {
  __shared__ __attribute__((aligned(16))) uint64_t cand[4][kTopkCand];
  __shared__ uint64_t sel[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;  // waves work independently (wave-private LDS, no barrier)
  const float* row = logits + (size_t)t * E;
  const uint64_t mine = topk_token<V>(row, E, k, cand[wv], sel[wv], sel_bias);
  const float g = sel_bias ? topk_gate_unbiased(mine, k, row) : topk_gate_of(mine, k);
  if (lane < k) {
    idx[(size_t)t * k + lane] = topk_key_index(mine);
    gate[(size_t)t * k + lane] = g;
  }
}

hipError_t launch_topk(const float* logits, int T, const Shape& s, const float* sel_bias,
                       int32_t* idx, float* gate, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  dim3 grid((T + 3) / 4);
  if (s.E <= 256)
    hipLaunchKernelGGL(topk_kernel<4>, grid, dim3(256), 0, st, logits, T, s.E, s.k, sel_bias, idx,
                       gate);
  else if (s.E <= 1024)
    hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(256), 0, st, logits, T, s.E, s.k, sel_bias, idx,
                       gate);
  else
    hipLaunchKernelGGL(topk_kernel<64>, grid, dim3(256), 0, st, logits, T, s.E, s.k, sel_bias, idx,
                       gate);
  return hipGetLastError();
}

}  // namespace k3
