// Decode path (few tokens): the expert FFNs as bandwidth-bound MXFP4 GEMVs
// over the tiled MXFP4 layout (see layout.hip).
// Prior art: the pages' MXFP4 matmul works on the packed nibbles directly and
// never materialises a dequantised expert (kimi-k3-in-c CHANGELOG walk-through,
// 0.1.0 section). Here each lane loads whole 32-element MX blocks (16 bytes of
// E2M1 codes) with coalesced 16-byte loads (a wave reads one 1 KB tile),
// decodes nibble pairs in registers with the gfx950 FP4 converts,
// accumulates in fp32, applies the E8M0 block scale once per block and sums
// each row over its four lane groups.
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

// gate/up: one wave per (pair, 16-row tile of gate and of up). Lane (r, g)
// takes row 16 rt + r, K block g of every 128-column tile, so one 16-byte
// load per lane reads a whole 1 KB tile; its 32 activations are the same for
// the 16 lanes of a group (a broadcast load). Rows are summed over the 4
// groups at the end. Four K tiles per step share one scale dword per lane.
// grid: (T*k pairs, ceil(f / 64)), block 256 (4 waves = 4 row tiles).
__global__ __launch_bounds__(256) void gemv_gateup_kernel(
    const uint16_t* __restrict__ x, int d, int f, int k, int E, const uint8_t* __restrict__ gq,
    const uint8_t* __restrict__ gs, const uint8_t* __restrict__ uq, const uint8_t* __restrict__ us,
    const int32_t* __restrict__ idx, float* __restrict__ h32) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int pair = blockIdx.x;
  const int rt = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int RT = f >> 4, KT = d >> 7, KG = (KT + 3) >> 2;
  if (rt >= RT) return;
  const int t = pair / k;
  const int e = idx[pair];
  if (e < 0 || e >= E) return;  // dropped pair: never read downstream
  const size_t tile0 = ((size_t)e * RT + rt) * KT;
  const uint8_t* gqt = gq + tile0 * 1024 + 16 * lane;
  const uint8_t* uqt = uq + tile0 * 1024 + 16 * lane;
  const size_t grp0 = ((size_t)e * RT + rt) * KG;
  const uint32_t* gst = reinterpret_cast<const uint32_t*>(gs + grp0 * 256) + lane;
  const uint32_t* ust = reinterpret_cast<const uint32_t*>(us + grp0 * 256) + lane;
  const uint16_t* xt = x + (size_t)t * d + 32 * g;
  float ga = 0.0f, ua = 0.0f;
  for (int kg = 0; kg < KG; ++kg) {
    const uint32_t sgw = gst[64 * kg], suw = ust[64 * kg];
    const int nk = min(4, KT - 4 * kg);
    uint4 qg[4], qu[4];
    uint32_t xr[4][16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < nk) {
        const int kt = 4 * kg + j;
        qg[j] = *reinterpret_cast<const uint4*>(gqt + (size_t)kt * 1024);
        qu[j] = *reinterpret_cast<const uint4*>(uqt + (size_t)kt * 1024);
        const uint4* xs = reinterpret_cast<const uint4*>(xt + 128 * kt);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 q = xs[v];
          xr[j][4 * v] = q.x; xr[j][4 * v + 1] = q.y; xr[j][4 * v + 2] = q.z; xr[j][4 * v + 3] = q.w;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < nk) {
        ga = fmaf(block_dot_bf16(qg[j], xr[j]), e8m0_to_f32((sgw >> (8 * j)) & 0xffu), ga);
        ua = fmaf(block_dot_bf16(qu[j], xr[j]), e8m0_to_f32((suw >> (8 * j)) & 0xffu), ua);
      }
    }
  }
  ga += __shfl_xor(ga, 16, 64);
  ga += __shfl_xor(ga, 32, 64);
  ua += __shfl_xor(ua, 16, 64);
  ua += __shfl_xor(ua, 32, 64);
  if (g == 0) h32[(size_t)pair * f + 16 * rt + r] = silu_f32(ga) * ua;
}

// down + combine: workgroup = one token x one 16-row tile of the output; its
// 8 waves split the token's k slots (wave w: j = w, w + 8, ...). For each
// slot a wave issues the loads of all its K tiles (the next slot's are issued
// before the current one is computed), stages the pair's h (fp32) in its own
// LDS region and reads each 32-value block of it as a broadcast. Lane (r, g)
// keeps a gate-weighted partial of row 16 rt + r over K block g of every
// tile; partials meet across lane groups, then across waves in fixed order.
// Deterministic, no atomics.
// grid: (T, d / 16), block 512, dynamic LDS 32 f bytes.
constexpr int kDownTiles = 4;  // K tiles per step (a slot of f = 2048 takes 4 steps)
constexpr int kDownWaves = 8;
__global__ __launch_bounds__(64 * kDownWaves) void gemv_down_kernel(
    int d, int f, int k, int E, const uint8_t* __restrict__ dq, const uint8_t* __restrict__ ds,
    const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const float* __restrict__ h32, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) float hl[];  // [kDownWaves][f]
  __shared__ float red[kDownWaves][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int t = blockIdx.x, rt = blockIdx.y;
  const int RT = d >> 4, KT = f >> 7, KG = (KT + 3) >> 2;
  float* hw = hl + (size_t)wave * f;
  struct Slot {
    uint4 q[kDownTiles];
    uint32_t sw[kDownTiles / 4];
  };
  // loads of K tiles kt0 .. kt0 + 15 of slot j's expert (nothing for a
  // dropped slot)
  auto issue = [&](int j, int kt0, Slot& sl) {
    const int e = idx[(size_t)t * k + j];
    if (e < 0 || e >= E) return;
    const size_t tile0 = ((size_t)e * RT + rt) * KT;
    const uint8_t* qt = dq + tile0 * 1024 + 16 * lane;
    const uint32_t* st = reinterpret_cast<const uint32_t*>(ds + ((size_t)e * RT + rt) * KG * 256) + lane;
    const int n = min(kDownTiles, KT - kt0);
#pragma unroll
    for (int i = 0; i < kDownTiles; ++i)
      if (i < n) sl.q[i] = *reinterpret_cast<const uint4*>(qt + (size_t)(kt0 + i) * 1024);
#pragma unroll
    for (int s2 = 0; s2 < kDownTiles / 4; ++s2)
      if (4 * s2 < n) sl.sw[s2] = st[64 * ((kt0 >> 2) + s2)];
  };
  float acc = 0.0f;
  // h of slot j: its first 2048 values go through registers (loaded before
  // the next step's weights, so waiting for them does not wait for those),
  // the rest (f > 2048) straight into LDS
  constexpr int kStageF4 = 8;  // float4 per lane held in registers
  const int n4 = f >> 2;
  auto compute = [&](int j, int kt0, const Slot& sl) {
    const int pair = t * k + j;
    const int n = min(kDownTiles, KT - kt0);
    float pe = 0.0f;
#pragma unroll
    for (int i = 0; i < kDownTiles; ++i)
      if (i < n) {
        const float4* hs = reinterpret_cast<const float4*>(hw + 128 * (kt0 + i) + 32 * g);
        float hv[32];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float4 h4 = hs[v];
          hv[4 * v] = h4.x; hv[4 * v + 1] = h4.y; hv[4 * v + 2] = h4.z; hv[4 * v + 3] = h4.w;
        }
        pe = fmaf(block_dot_f32(sl.q[i], hv),
                  e8m0_to_f32((sl.sw[i >> 2] >> (8 * (i & 3))) & 0xffu), pe);
      }
    acc = fmaf(gate[pair], pe, acc);
  };
  auto valid = [&](int j) {
    const int e = idx[(size_t)t * k + j];
    return e >= 0 && e < E;  // a dropped pair contributes zero
  };
  // the wave's (slot, 16-tile chunk) steps; step s+1's weights are issued
  // after step s's h is loaded and before step s is computed
  const int nchunk = (KT + kDownTiles - 1) / kDownTiles;
  const int nslot = (k - wave + kDownWaves - 1) / kDownWaves;  // slots wave, wave + 8, ...
  const int nstep = nslot * nchunk;
  Slot sa, sb;
  auto step = [&](int s, Slot& cur, Slot& nxt) {
    const int j = wave + kDownWaves * (s / nchunk), kt0 = kDownTiles * (s % nchunk);
    const bool on = valid(j);
    const bool stage = on && kt0 == 0;
    const float4* hsrc = reinterpret_cast<const float4*>(h32 + (size_t)(t * k + j) * f);
    float4 hr0, hr1, hr2, hr3, hr4, hr5, hr6, hr7;  // lane + 64 v, v = 0..7 (clamped)
    if (stage) {
      hr0 = hsrc[min(lane, n4 - 1)];
      hr1 = hsrc[min(lane + 64, n4 - 1)];
      hr2 = hsrc[min(lane + 128, n4 - 1)];
      hr3 = hsrc[min(lane + 192, n4 - 1)];
      hr4 = hsrc[min(lane + 256, n4 - 1)];
      hr5 = hsrc[min(lane + 320, n4 - 1)];
      hr6 = hsrc[min(lane + 384, n4 - 1)];
      hr7 = hsrc[min(lane + 448, n4 - 1)];
    }
    if (s + 1 < nstep)
      issue(wave + kDownWaves * ((s + 1) / nchunk), kDownTiles * ((s + 1) % nchunk), nxt);
    if (!on) return;
    if (stage) {
      float4* hd = reinterpret_cast<float4*>(hw);
      if (lane < n4) hd[lane] = hr0;
      if (lane + 64 < n4) hd[lane + 64] = hr1;
      if (lane + 128 < n4) hd[lane + 128] = hr2;
      if (lane + 192 < n4) hd[lane + 192] = hr3;
      if (lane + 256 < n4) hd[lane + 256] = hr4;
      if (lane + 320 < n4) hd[lane + 320] = hr5;
      if (lane + 384 < n4) hd[lane + 384] = hr6;
      if (lane + 448 < n4) hd[lane + 448] = hr7;
      for (int i = lane + 64 * kStageF4; i < n4; i += 64) hd[i] = hsrc[i];
    }
    compute(j, kt0, cur);
  };
  if (nstep > 0) issue(wave, 0, sa);
  for (int s = 0; s < nstep; s += 2) {
    step(s, sa, sb);
    if (s + 1 < nstep) step(s + 1, sb, sa);
  }
  acc += __shfl_xor(acc, 16, 64);
  acc += __shfl_xor(acc, 32, 64);
  if (g == 0) red[wave][r] = acc;
  __syncthreads();
  if (tid < 16) {
    float s = red[0][tid];
#pragma unroll
    for (int w = 1; w < kDownWaves; ++w) s += red[w][tid];
    y[(size_t)t * d + 16 * rt + tid] = s;
  }
}

hipError_t launch_gemv_gateup(const uint16_t* x, int T, const Shape& s, const ExpertWeights& w,
                              const int32_t* idx, float* h32, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  dim3 g1(T * s.k, (s.f / 16 + 3) / 4);
  hipLaunchKernelGGL(gemv_gateup_kernel, g1, dim3(256), 0, st, x, s.d, s.f, s.k, s.E, w.gate_q,
                     w.gate_s, w.up_q, w.up_s, idx, h32);
  return hipGetLastError();
}

hipError_t prepare_gemv(const Shape& s) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_down_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, 4 * kDownWaves * s.f);
}

hipError_t launch_gemv_down(int T, const Shape& s, const ExpertWeights& w, const int32_t* idx,
                            const float* gate, const float* h32, float* y, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  dim3 g2(T, s.d / 16);
  hipLaunchKernelGGL(gemv_down_kernel, g2, dim3(64 * kDownWaves), (size_t)4 * kDownWaves * s.f, st,
                     s.d, s.f, s.k, s.E,
                     w.down_q, w.down_s, idx, gate, h32, y);
  return hipGetLastError();
}

}  // namespace k3
