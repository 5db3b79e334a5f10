// Decode path (few tokens): the expert FFNs as bandwidth-bound MXFP4 GEMVs.
// Prior art: the pages' MXFP4 matmul works on the packed nibbles directly and
// never materialises a dequantised expert (kimi-k3-in-c CHANGELOG walk-through,
// 0.1.0 section). Here each lane loads whole 32-element MX blocks (16 bytes of
// E2M1 codes + 1 E8M0 byte) with coalesced 16-byte loads, decodes nibble
// pairs in registers with the gfx950 FP4->bf16 convert, accumulates with
// bf16 dot products into fp32, applies the block scale once per block and
// reduces across the wave.
//
//   gemv_gateup: per (token, slot) pair and feature n:
//       g = Wg[e][n,:] . x,  u = Wu[e][n,:] . x,  h[n] = SiLU(g) * u   (fp32)
//   gemv_down:   per token and output row m:
//       y[m] = sum_j gate_j * (Wd[e_j][m,:] . h_j)                        (fp32)
// Both are deterministic (fixed summation order, no atomics).
#include "k3_device.h"
#include "k3_kernels.h"

namespace k3 {

// Dot product of one 32-element MX block of codes (4 dwords) with 32 bf16
// activations (16 packed pairs), fp32 result before the block scale.
__device__ __forceinline__ float block_dot_bf16(const uint4 q, const uint32_t* xp) {
  float acc = 0.0f;
  const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    v2bf a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(qw[w], 1.0f, 0);
    v2bf a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(qw[w], 1.0f, 1);
    v2bf a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(qw[w], 1.0f, 2);
    v2bf a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(qw[w], 1.0f, 3);
    acc = __builtin_amdgcn_fdot2_f32_bf16(a0, __builtin_bit_cast(v2bf, xp[4 * w + 0]), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(a1, __builtin_bit_cast(v2bf, xp[4 * w + 1]), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(a2, __builtin_bit_cast(v2bf, xp[4 * w + 2]), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(a3, __builtin_bit_cast(v2bf, xp[4 * w + 3]), acc, false);
  }
  return acc;
}

// Dot product of one MX block of codes with 32 fp32 values (h), fp32.
__device__ __forceinline__ float block_dot_f32(const uint4 q, const float* hv) {
  float acc = 0.0f;
  const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    v2f a0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qw[w], 1.0f, 0);
    v2f a1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qw[w], 1.0f, 1);
    v2f a2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qw[w], 1.0f, 2);
    v2f a3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qw[w], 1.0f, 3);
    acc = fmaf(a0[0], hv[8 * w + 0], acc);
    acc = fmaf(a0[1], hv[8 * w + 1], acc);
    acc = fmaf(a1[0], hv[8 * w + 2], acc);
    acc = fmaf(a1[1], hv[8 * w + 3], acc);
    acc = fmaf(a2[0], hv[8 * w + 4], acc);
    acc = fmaf(a2[1], hv[8 * w + 5], acc);
    acc = fmaf(a3[0], hv[8 * w + 6], acc);
    acc = fmaf(a3[1], hv[8 * w + 7], acc);
  }
  return acc;
}

constexpr int kGateUpRowsPerWave = 4;

// grid: (T*k pairs, ceil(f / (4 * kGateUpRowsPerWave))), block 256.
// NBL = MX blocks of the reduction dim handled per lane (ceil((d/32)/64)).
template <int NBL>
__global__ __launch_bounds__(256) void gemv_gateup_kernel(
    const uint16_t* __restrict__ x, int d, int f, int k, int E, const uint8_t* __restrict__ gq,
    const uint8_t* __restrict__ gs, const uint8_t* __restrict__ uq, const uint8_t* __restrict__ us,
    const int32_t* __restrict__ idx, float* __restrict__ h32) {
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x;
  const int t = pair / k;
  const int e = idx[pair];
  if (e < 0 || e >= E) return;  // dropped pair: never read downstream
  const int nb = d >> 5;
  // activations of this lane's blocks, as packed bf16 pairs
  uint32_t xr[NBL][16];
#pragma unroll
  for (int b = 0; b < NBL; ++b) {
    const int blk = lane + 64 * b;
    if (blk < nb) {
      const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * d + 32 * blk);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        uint4 q = src[v];
        xr[b][4 * v + 0] = q.x; xr[b][4 * v + 1] = q.y; xr[b][4 * v + 2] = q.z; xr[b][4 * v + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) xr[b][v] = 0u;
    }
  }
  const int n0 = (blockIdx.y * 4 + (threadIdx.x >> 6)) * kGateUpRowsPerWave;
  const size_t qrow = (size_t)(d >> 1), srow = (size_t)nb;
  // two row pairs per pass; all of a pass's loads are issued before any math
#pragma unroll
  for (int r0 = 0; r0 < kGateUpRowsPerWave; r0 += 2) {
    uint4 qg[2][NBL], qu[2][NBL];
    uint32_t sg[2][NBL], su[2][NBL];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int n = min(n0 + r0 + rr, f - 1);
      const size_t row = (size_t)e * f + n;
#pragma unroll
      for (int b = 0; b < NBL; ++b) {
        const int blk = lane + 64 * b;
        if (blk < nb) {
          qg[rr][b] = *reinterpret_cast<const uint4*>(gq + row * qrow + 16 * blk);
          qu[rr][b] = *reinterpret_cast<const uint4*>(uq + row * qrow + 16 * blk);
          sg[rr][b] = gs[row * srow + blk];
          su[rr][b] = us[row * srow + blk];
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int n = n0 + r0 + rr;
      float ga = 0.0f, ua = 0.0f;
#pragma unroll
      for (int b = 0; b < NBL; ++b) {
        const int blk = lane + 64 * b;
        if (blk < nb) {
          ga = fmaf(block_dot_bf16(qg[rr][b], xr[b]), e8m0_to_f32(sg[rr][b]), ga);
          ua = fmaf(block_dot_bf16(qu[rr][b], xr[b]), e8m0_to_f32(su[rr][b]), ua);
        }
      }
      ga = wave_sum(ga);
      ua = wave_sum(ua);
      if (lane == 0 && n < f) h32[(size_t)pair * f + n] = silu_f32(ga) * ua;
    }
  }
}

constexpr int kDownRowsPerBlock = 16;

// grid: (T, ceil(d / kDownRowsPerBlock)), block 256 (4 waves). Wave w handles
// slots j = w, w+4, ... of the token for all kDownRowsPerBlock rows; lanes
// keep gate-weighted partials, reduced once at the end, then the 4 waves are
// summed in fixed order through LDS.
template <int NBF>
__global__ __launch_bounds__(256) void gemv_down_kernel(
    int d, int f, int k, int E, const uint8_t* __restrict__ dq, const uint8_t* __restrict__ ds,
    const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const float* __restrict__ h32, float* __restrict__ y) {
  __shared__ float part[4][kDownRowsPerBlock];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x;
  const int m0 = blockIdx.y * kDownRowsPerBlock;
  const int nbf = f >> 5;
  const size_t qrow = (size_t)(f >> 1), srow = (size_t)nbf;
  float acc[kDownRowsPerBlock];
#pragma unroll
  for (int r = 0; r < kDownRowsPerBlock; ++r) acc[r] = 0.0f;
  for (int j = wave; j < k; j += 4) {
    const int pair = t * k + j;
    const int e = idx[pair];
    if (e < 0 || e >= E) continue;  // dropped pair contributes zero
    const float g = gate[pair];
    float hv[NBF][32];
#pragma unroll
    for (int b = 0; b < NBF; ++b) {
      const int blk = lane + 64 * b;
      if (blk < nbf) {
        const float4* src = reinterpret_cast<const float4*>(h32 + (size_t)pair * f + 32 * blk);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          float4 q = src[v];
          hv[b][4 * v] = q.x; hv[b][4 * v + 1] = q.y; hv[b][4 * v + 2] = q.z; hv[b][4 * v + 3] = q.w;
        }
      }
    }
    // all rows' loads first, then the math
    uint4 q[kDownRowsPerBlock][NBF];
    uint32_t sc[kDownRowsPerBlock][NBF];
#pragma unroll
    for (int r = 0; r < kDownRowsPerBlock; ++r) {
      const size_t row = (size_t)e * d + min(m0 + r, d - 1);
#pragma unroll
      for (int b = 0; b < NBF; ++b) {
        const int blk = lane + 64 * b;
        if (blk < nbf) {
          q[r][b] = *reinterpret_cast<const uint4*>(dq + row * qrow + 16 * blk);
          sc[r][b] = ds[row * srow + blk];
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kDownRowsPerBlock; ++r) {
#pragma unroll
      for (int b = 0; b < NBF; ++b) {
        const int blk = lane + 64 * b;
        if (blk < nbf) acc[r] = fmaf(g * e8m0_to_f32(sc[r][b]), block_dot_f32(q[r][b], hv[b]), acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kDownRowsPerBlock; ++r) {
    float s = wave_sum(acc[r]);
    if (lane == 0) part[wave][r] = s;
  }
  __syncthreads();
  if (threadIdx.x < kDownRowsPerBlock) {
    const int m = m0 + threadIdx.x;
    if (m < d) {
      float s = part[0][threadIdx.x];
      s += part[1][threadIdx.x];
      s += part[2][threadIdx.x];
      s += part[3][threadIdx.x];
      y[(size_t)t * d + m] = s;
    }
  }
}

hipError_t launch_gemv_gateup(const uint16_t* x, int T, const Shape& s, const ExpertWeights& w,
                              const int32_t* idx, float* h32, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const int nbl = (s.d / 32 + 63) / 64;
  dim3 g1(T * s.k, (s.f + 4 * kGateUpRowsPerWave - 1) / (4 * kGateUpRowsPerWave));
#define K3_GU(N) hipLaunchKernelGGL(gemv_gateup_kernel<N>, g1, dim3(256), 0, st, x, s.d, s.f, s.k, s.E, \
                                    w.gate_q, w.gate_s, w.up_q, w.up_s, idx, h32)
  // d <= 8192: at most 4 blocks per lane
  if (nbl <= 1) K3_GU(1);
  else if (nbl <= 2) K3_GU(2);
  else K3_GU(4);
#undef K3_GU
  return hipGetLastError();
}

hipError_t launch_gemv_down(int T, const Shape& s, const ExpertWeights& w, const int32_t* idx,
                            const float* gate, const float* h32, float* y, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const int nbfl = (s.f / 32 + 63) / 64;
  dim3 g2(T, (s.d + kDownRowsPerBlock - 1) / kDownRowsPerBlock);
#define K3_DN(N) hipLaunchKernelGGL(gemv_down_kernel<N>, g2, dim3(256), 0, st, s.d, s.f, s.k, s.E, \
                                    w.down_q, w.down_s, idx, gate, h32, y)
  // f <= 4096: at most 2 blocks per lane
  if (nbfl <= 1) K3_DN(1);
  else K3_DN(2);
#undef K3_DN
  return hipGetLastError();
}

}  // namespace k3
