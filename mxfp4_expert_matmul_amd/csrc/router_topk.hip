// Router: fp32 logits l[t,e] = sum_i x[t,i] * Wr[e,i] (+ bias[e]), then per
// token the top-k experts by (logit descending, index ascending) and gates
// renormalised over the selection, gate_j = exp(l_j - l_max) / sum_S exp(.).
// (kimi-k3-in-c CHANGELOG walk-through, 0.1.0 section: the MoE router picks
// top-16 of 896 routed experts; scoring and normalisation are not given on
// the pages and follow the plainest reading.)
#include "k3_device.h"
#include "k3_kernels.h"

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
// Tiled fp32 GEMM: 64 tokens x 64 experts per workgroup, K staged in LDS in
// steps of 32; each thread owns a 4x4 block of outputs.
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x, int T,
                                                          int d, const float* __restrict__ wr,
                                                          const float* __restrict__ bias, int E,
                                                          float* __restrict__ logits) {
  __shared__ float xs[32][64 + 4];  // [k][token]
  __shared__ float ws[32][64 + 4];  // [k][expert]
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tr = (tid >> 4) * 4;  // token offset in tile
  const int er = (tid & 15) * 4;  // expert offset in tile
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += 32) {
    // load 64x32 of x (bf16) and 64x32 of wr: 2048 elements each, 8 per thread
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      int li = tid + 256 * r;  // 0..2047
      int row = li >> 5, kk = li & 31;
      int t = t0 + row, e = e0 + row;
      xs[kk][row] = (t < T) ? bf16_bits_to_f32(x[(size_t)t * d + k0 + kk]) : 0.0f;
      ws[kk][row] = (e < E) ? wr[(size_t)e * d + k0 + kk] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = xs[kk][tr + i]; b[i] = ws[kk][er + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int t = t0 + tr + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = e0 + er + j;
      if (e < E) logits[(size_t)t * E + e] = acc[i][j] + (bias ? bias[e] : 0.0f);
    }
  }
}

hipError_t launch_router_logits(const uint16_t* x, int T, const Shape& s, const float* wr,
                                const float* bias, float* logits, hipStream_t st) {
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
    hipLaunchKernelGGL(router_gemm_kernel, grid, dim3(256), 0, st, x, T, s.d, wr, bias, s.E, logits);
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
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off, 64);
      int oi = __shfl_xor(bi, off, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
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
