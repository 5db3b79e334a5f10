// Router: fp32 logits l[t,e] = sum_i x[t,i] * Wr[e,i] (+ bias[e]), then per
// token the top-k experts by (logit descending, index ascending) and gates
// renormalised over the selection, gate_j = exp(l_j - l_max) / sum_S exp(.).
// (kimi-k3-in-c CHANGELOG walk-through, 0.1.0 section: the MoE router picks
// top-16 of 896 routed experts; scoring and normalisation are not given on
// the pages and follow the plainest reading.)
#include "k3_device.h"
#include "k3_kernels.h"

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
  float4 w[kMaxPer];
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const int i = tid + 256 * j;
    if (i < n4) w[j] = row[i];
  }
  float acc[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) acc[t] = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const int i = tid + 256 * j;
    if (i < n4) {
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        if (t < T) {
          uint2 xv = *reinterpret_cast<const uint2*>(x + (size_t)t * d + 4 * i);
          acc[t] = fmaf(bf16_bits_to_f32(xv.x & 0xffffu), w[j].x, acc[t]);
          acc[t] = fmaf(bf16_bits_to_f32(xv.x >> 16), w[j].y, acc[t]);
          acc[t] = fmaf(bf16_bits_to_f32(xv.y & 0xffffu), w[j].z, acc[t]);
          acc[t] = fmaf(bf16_bits_to_f32(xv.y >> 16), w[j].w, acc[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if (t < T) {
      float s = wave_sum(acc[t]);
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

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

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

// grid: (ceil(T / 64), ceil(E / 64)), block 256. Wave w owns experts
// e0 + 16 w .. +15 (MFMA rows) for tokens t0 .. t0 + 63 (four 16-column tiles).
// MFMA operand lane l: row/column l % 16, 8 consecutive K at 8 (l / 16); both
// operands use the same layout, so any consistent K order is a valid sum.
__global__ __launch_bounds__(256) void router_mfma_kernel(const uint16_t* __restrict__ x, int T,
                                                          int d, const uint16_t* __restrict__ w3,
                                                          const float* __restrict__ bias, int E,
                                                          float* __restrict__ logits) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64 + 16 * wave;
  const size_t n = (size_t)E * d;
  const int ea = min(e0 + r, E - 1);
  const uint16_t* ap = w3 + (size_t)ea * d + 8 * g;
  const uint16_t* bp[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) bp[ct] = x + (size_t)min(t0 + 16 * ct + r, T - 1) * d + 8 * g;
  v4f acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int k0 = 0; k0 < d; k0 += 32) {
    v8bf a[3], b[4];
#pragma unroll
    for (int q = 0; q < 3; ++q) a[q] = *reinterpret_cast<const v8bf*>(ap + q * n + k0);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) b[ct] = *reinterpret_cast<const v8bf*>(bp[ct] + k0);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int q = 0; q < 3; ++q)
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q], b[ct], acc[ct], 0, 0, 0);
  }
  // result element i of lane l: expert e0 + 4 g + i, token t0 + 16 ct + r
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int t = t0 + 16 * ct + r;
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + 4 * g + i;
      if (e < E) logits[(size_t)t * E + e] = acc[ct][i] + (bias ? bias[e] : 0.0f);
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
    dim3 grid((T + 63) / 64, (s.E + 63) / 64);
    hipLaunchKernelGGL(router_mfma_kernel, grid, dim3(256), 0, st, x, T, s.d, wr3, bias, s.E, logits);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- top-k + gates
// One wave per token; the token's logits are read once into registers. Round
// r selects the best element strictly below the previous selection in the
// order (value descending, index ascending), so no mask is needed; NaN ranks
// as -inf so a valid index is always chosen.
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// One DPP step of the arg-max reduction: combine with the lane selected by
// CTRL (row_mask selects the 16-lane rows that take part; others keep their
// own pair).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
  const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, ROW_MASK, 0xf, false);
  if (better(ov, oi, v, i)) { v = ov; i = oi; }
}

// Arg-max over the 64 lanes in the order (value descending, index ascending):
// quad swaps, half-row and row mirrors give every lane its 16-lane row's best;
// row broadcasts of lanes 15 and 31 carry the rows forward so lane 63 holds
// the wave's best, which is then read by every lane.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<0xB1, 0xf>(v, i);   // quad_perm [1,0,3,2]
  argmax_step<0x4E, 0xf>(v, i);   // quad_perm [2,3,0,1]
  argmax_step<0x141, 0xf>(v, i);  // row_half_mirror
  argmax_step<0x140, 0xf>(v, i);  // row_mirror
  argmax_step<0x142, 0xa>(v, i);  // row_bcast15 into rows 1 and 3
  argmax_step<0x143, 0xc>(v, i);  // row_bcast31 into rows 2 and 3
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

template <int V>  // logits per lane: E <= 64 * V
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  const float NEG_INF = -__builtin_huge_valf();
  float v[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int e = lane + 64 * j;
    float a = (e < E) ? row[e] : NEG_INF;
    v[j] = (a != a) ? NEG_INF : a;  // NaN ranks as -inf
  }
  float pv = __builtin_huge_valf();  // previous selection (value, index)
  int pi = -1;
  float myv = NEG_INF;  // lane r keeps the value of selection r
  for (int r = 0; r < k; ++r) {
    float bv = NEG_INF;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int e = lane + 64 * j;
      const bool below = (v[j] < pv) || (v[j] == pv && e > pi);
      if (e < E && below && better(v[j], e, bv, bi)) { bv = v[j]; bi = e; }
    }
    wave_argmax(bv, bi);  // every lane gets the wave's best (value, index)
    pv = bv;
    pi = bi;
    if (lane == r) myv = bv;
    if (lane == 0) idx[(size_t)t * k + r] = bi;
  }
  const float vmax = __shfl(myv, 0, 64);
  float w = (lane < k) ? expf(myv - vmax) : 0.0f;
  const float sum = wave_sum(w);
  if (lane < k) gate[(size_t)t * k + lane] = w / sum;
}

hipError_t launch_topk(const float* logits, int T, const Shape& s, int32_t* idx, float* gate,
                       hipStream_t st) {
  if (T <= 0) return hipSuccess;
  dim3 grid((T + 3) / 4);
  if (s.E <= 256)
    hipLaunchKernelGGL(topk_kernel<4>, grid, dim3(256), 0, st, logits, T, s.E, s.k, idx, gate);
  else if (s.E <= 1024)
    hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(256), 0, st, logits, T, s.E, s.k, idx, gate);
  else
    hipLaunchKernelGGL(topk_kernel<64>, grid, dim3(256), 0, st, logits, T, s.E, s.k, idx, gate);
  return hipGetLastError();
}

}  // namespace k3
