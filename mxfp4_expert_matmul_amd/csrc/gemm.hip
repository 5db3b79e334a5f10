// Prefill path: grouped GEMMs on the gfx950 scaled MX MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4). Expert weights enter the MFMA as
// native MXFP4 (E2M1 codes + their own E8M0 block scales), never dequantised;
// this is the GPU counterpart of the pages' MXFP4 matmul that consumes packed
// nibbles directly (kimi-k3-in-c CHANGELOG walk-through, 0.1.0 section).
// Tokens are grouped per expert first (chunk-union prefill, Unreleased
// section), so one tile reads an expert's weight rows once for up to
// kTileM tokens.
//
// Activations are bf16 and must reach the MFMA without losing precision, so
// each 32-element block of x is split into two E4M3 terms with their own E8M0
// scales, x ~= s1*hi + s2*lo, s1 = 2^(floor(log2 max|x|) - 7) (block max in
// [128, 256): no clamping), s2 from the block max of the residual; the pair
// reproduces bf16 blocks to within about 2^-16 of the block max. The SwiGLU
// output h (fp32) is split the same way before the down projection. Each
// term is one MFMA, accumulated in fp32.
//
// Operand lane layouts (measured on gfx950 for 16x16x128 f8f6f4):
//   lane l: row/column r = l % 16, lane group g = l / 16
//   FP4 operand: 16 bytes = K slots 32g .. 32g+31 (element 2i low nibble)
//   FP8 operand: bytes 0-15 = K slots 16g .. 16g+15,
//                bytes 16-31 = K slots 64+16g .. 64+16g+15
//   scale operand of lane l: row/column r, K slots 32g .. 32g+31
//   result: lane l, element i -> row 4g + i of A, column l % 16 of B
// The physical 32-element block behind MFMA slot-block kappa of step s of a
// super-step of S steps starting at block kb0 is kb0 + S*kappa + s, so one
// lane's S blocks of weights are contiguous (one 16*S-byte run per row).
#include "k3_device.h"
#include "k3_kernels.h"

namespace k3 {

constexpr int kFmtFp8 = 0;
constexpr int kFmtFp4 = 4;

// ------------------------------------------------------------- split of x
// One thread per 32-element block of x.
__global__ __launch_bounds__(256) void quant_x_kernel(const uint16_t* __restrict__ x, int nblk,
                                                      int nb, uint8_t* __restrict__ xq_hi,
                                                      uint8_t* __restrict__ xq_lo,
                                                      uint8_t* __restrict__ xs_hi,
                                                      uint8_t* __restrict__ xs_lo) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= nblk) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)i * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint4 w = src[q];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * q + 2 * j] = bf16_bits_to_f32(ww[j] & 0xffffu);
      v[8 * q + 2 * j + 1] = bf16_bits_to_f32(ww[j] >> 16);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const uint32_t b1 = e4m3_block_scale_byte(amax);
  const float s1 = e8m0_to_f32(b1), s1inv = e8m0_to_f32(254u - b1);
  float hi[32], r[32];
  float ramax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    hi[j] = round_e4m3(v[j] * s1inv);
    r[j] = v[j] - hi[j] * s1;
    ramax = fmaxf(ramax, fabsf(r[j]));
  }
  const uint32_t b2 = e4m3_block_scale_byte(ramax);
  const float s2inv = e8m0_to_f32(254u - b2);
  uint32_t ph[8], pl[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    ph[q] = pack4_e4m3(hi[4 * q], hi[4 * q + 1], hi[4 * q + 2], hi[4 * q + 3]);
    pl[q] = pack4_e4m3(round_e4m3(r[4 * q] * s2inv), round_e4m3(r[4 * q + 1] * s2inv),
                       round_e4m3(r[4 * q + 2] * s2inv), round_e4m3(r[4 * q + 3] * s2inv));
  }
  uint4* dh = reinterpret_cast<uint4*>(xq_hi + (size_t)i * 32);
  uint4* dl = reinterpret_cast<uint4*>(xq_lo + (size_t)i * 32);
  dh[0] = make_uint4(ph[0], ph[1], ph[2], ph[3]);
  dh[1] = make_uint4(ph[4], ph[5], ph[6], ph[7]);
  dl[0] = make_uint4(pl[0], pl[1], pl[2], pl[3]);
  dl[1] = make_uint4(pl[4], pl[5], pl[6], pl[7]);
  xs_hi[i] = (uint8_t)b1;
  xs_lo[i] = (uint8_t)b2;
  (void)nb;
}

hipError_t launch_quant_x(const uint16_t* x, int T, int d, uint8_t* xq, uint8_t* xs,
                          hipStream_t st) {
  const int nb = d / 32;
  const int nblk = T * nb;
  if (nblk <= 0) return hipSuccess;
  const size_t plane = (size_t)T * d, splane = (size_t)T * nb;
  (void)plane;
  (void)splane;
  hipLaunchKernelGGL(quant_x_kernel, dim3((nblk + 255) / 256), dim3(256), 0, st, x, nblk, nb, xq,
                     xq + (size_t)T * d, xs, xs + (size_t)T * nb);
  return hipGetLastError();
}

// ------------------------------------------------------------- MFMA helpers
__device__ __forceinline__ v8i fp4_operand(const uint4 q) {
  v8i a = {(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
  return a;
}

__device__ __forceinline__ v8i fp8_operand(const uint4 lo, const uint4 hi) {
  v8i b = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  return b;
}

template <int OPSEL>
__device__ __forceinline__ v4f mfma_fp4_fp8(v8i a, int sa, v8i b, int sb, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kFmtFp4, kFmtFp8, OPSEL, sa,
                                                         OPSEL, sb);
}

// Tile geometry shared by both GEMMs: 4 waves; each wave owns 32 output rows
// of the weight matrix (two 16-row MFMA tiles) for up to 64 tokens (four
// 16-column MFMA tiles); a workgroup covers 128 weight rows.
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerBlock = 128;
constexpr int kColTiles = kTileM / 16;

struct TileInfo {
  int e, row0, cnt, base;  // expert, first sorted row in the expert, tokens, offsets[e]
};

__device__ __forceinline__ bool load_tile(const int32_t* tiles, const int32_t* ntiles,
                                          const int32_t* offsets, TileInfo& ti) {
  const int tile = blockIdx.x;
  if (tile >= ntiles[0]) return false;
  ti.e = tiles[2 * tile];
  ti.row0 = tiles[2 * tile + 1];
  ti.base = offsets[ti.e];
  const int total = offsets[ti.e + 1] - ti.base;
  ti.cnt = min(total - ti.row0, kTileM);
  return ti.cnt > 0;
}

// One super-step (S MFMA steps, 4*S blocks of K) for NM weight matrices of
// one wave: A rows (per matrix NRT row tiles), B = 2-term FP8 activations for
// up to kColTiles column tiles.
//   arow[mat][rt]  : byte pointer to this lane's weight row codes
//   asrow[mat][rt] : byte pointer to this lane's weight row scales
//   brow_hi/lo[ct] : byte pointer to this lane's activation row (hi / lo)
//   bs_hi/lo[ct]   : byte pointer to this lane's activation scale row
template <int S, int NM, int NRT>
__device__ __forceinline__ void mx_superstep(int kb0, int g, int nct,
                                             const uint8_t* const (&arow)[NM][NRT],
                                             const uint8_t* const (&asrow)[NM][NRT],
                                             const uint8_t* const (&brow_hi)[kColTiles],
                                             const uint8_t* const (&brow_lo)[kColTiles],
                                             const uint8_t* const (&bs_hi)[kColTiles],
                                             const uint8_t* const (&bs_lo)[kColTiles],
                                             v4f (&acc)[NM][NRT][kColTiles]) {
  // weights: S contiguous blocks per lane per row tile
  uint4 aq[NM][NRT][S];
  int as[NM][NRT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const uint4* p = reinterpret_cast<const uint4*>(arow[m][rt] + 16 * (kb0 + S * g));
#pragma unroll
      for (int s = 0; s < S; ++s) aq[m][rt][s] = p[s];
      if (S == 4)
        as[m][rt] = *reinterpret_cast<const int*>(asrow[m][rt] + kb0 + 4 * g);
      else
        as[m][rt] = asrow[m][rt][kb0 + g];
    }
  int bsh[kColTiles], bsl[kColTiles];
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
    if (ct < nct) {
      if (S == 4) {
        bsh[ct] = *reinterpret_cast<const int*>(bs_hi[ct] + kb0 + 4 * g);
        bsl[ct] = *reinterpret_cast<const int*>(bs_lo[ct] + kb0 + 4 * g);
      } else {
        bsh[ct] = bs_hi[ct][kb0 + g];
        bsl[ct] = bs_lo[ct][kb0 + g];
      }
    }
  }
  const int half = 16 * (g & 1);
  const int b0 = kb0 + S * (g >> 1);      // slot-block g/2
  const int b1 = kb0 + S * (2 + (g >> 1));  // slot-block 2 + g/2
#pragma unroll
  for (int s = 0; s < S; ++s) {
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) {
      if (ct < nct) {
        const uint4 h0 = *reinterpret_cast<const uint4*>(brow_hi[ct] + 32 * (b0 + s) + half);
        const uint4 h1 = *reinterpret_cast<const uint4*>(brow_hi[ct] + 32 * (b1 + s) + half);
        const uint4 l0 = *reinterpret_cast<const uint4*>(brow_lo[ct] + 32 * (b0 + s) + half);
        const uint4 l1 = *reinterpret_cast<const uint4*>(brow_lo[ct] + 32 * (b1 + s) + half);
        const v8i bh = fp8_operand(h0, h1), bl = fp8_operand(l0, l1);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            const v8i a = fp4_operand(aq[m][rt][s]);
            if (S == 4) {
              if (s == 0) {
                acc[m][rt][ct] = mfma_fp4_fp8<0>(a, as[m][rt], bh, bsh[ct], acc[m][rt][ct]);
                acc[m][rt][ct] = mfma_fp4_fp8<0>(a, as[m][rt], bl, bsl[ct], acc[m][rt][ct]);
              } else if (s == 1) {
                acc[m][rt][ct] = mfma_fp4_fp8<1>(a, as[m][rt], bh, bsh[ct], acc[m][rt][ct]);
                acc[m][rt][ct] = mfma_fp4_fp8<1>(a, as[m][rt], bl, bsl[ct], acc[m][rt][ct]);
              } else if (s == 2) {
                acc[m][rt][ct] = mfma_fp4_fp8<2>(a, as[m][rt], bh, bsh[ct], acc[m][rt][ct]);
                acc[m][rt][ct] = mfma_fp4_fp8<2>(a, as[m][rt], bl, bsl[ct], acc[m][rt][ct]);
              } else {
                acc[m][rt][ct] = mfma_fp4_fp8<3>(a, as[m][rt], bh, bsh[ct], acc[m][rt][ct]);
                acc[m][rt][ct] = mfma_fp4_fp8<3>(a, as[m][rt], bl, bsl[ct], acc[m][rt][ct]);
              }
            } else {
              acc[m][rt][ct] = mfma_fp4_fp8<0>(a, as[m][rt], bh, bsh[ct], acc[m][rt][ct]);
              acc[m][rt][ct] = mfma_fp4_fp8<0>(a, as[m][rt], bl, bsl[ct], acc[m][rt][ct]);
            }
          }
      }
    }
  }
}

// ------------------------------------------------------------- gate/up + SwiGLU
// grid: (max_tiles, f / 128), block 256. Writes h for the tile's sorted rows
// as two E4M3 terms + E8M0 scales per 32 features: hq_hi/lo [P][f],
// hs_hi/lo [P][f/32].
__global__ __launch_bounds__(256) void gemm_gateup_kernel(
    int d, int f, int k, const uint8_t* __restrict__ gq, const uint8_t* __restrict__ gs,
    const uint8_t* __restrict__ uq, const uint8_t* __restrict__ us,
    const uint8_t* __restrict__ xq_hi, const uint8_t* __restrict__ xq_lo,
    const uint8_t* __restrict__ xs_hi, const uint8_t* __restrict__ xs_lo,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ ntiles,
    uint8_t* __restrict__ hq_hi, uint8_t* __restrict__ hq_lo, uint8_t* __restrict__ hs_hi,
    uint8_t* __restrict__ hs_lo) {
  TileInfo ti;
  if (!load_tile(tiles, ntiles, offsets, ti)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int nb = d >> 5, nbf = f >> 5;
  const int nct = (ti.cnt + 15) >> 4;
  const int nw0 = blockIdx.y * kRowsPerBlock + wave * kRowsPerWave;  // first feature of the wave
  // weight row pointers: matrix 0 = gate, 1 = up; row tile rt covers nw0 + 16 rt + (0..15)
  const uint8_t* arow[2][2];
  const uint8_t* asrow[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const size_t row = (size_t)ti.e * f + nw0 + 16 * rt + r;
    arow[0][rt] = gq + row * (size_t)(d >> 1);
    arow[1][rt] = uq + row * (size_t)(d >> 1);
    asrow[0][rt] = gs + row * (size_t)nb;
    asrow[1][rt] = us + row * (size_t)nb;
  }
  // activation rows of this lane's token in each column tile
  const uint8_t* bh[kColTiles];
  const uint8_t* bl[kColTiles];
  const uint8_t* bsh[kColTiles];
  const uint8_t* bsl[kColTiles];
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
    int i = 16 * ct + r;
    if (i >= ti.cnt) i = 0;
    const int tok = perm[ti.base + ti.row0 + i] / k;
    bh[ct] = xq_hi + (size_t)tok * d;
    bl[ct] = xq_lo + (size_t)tok * d;
    bsh[ct] = xs_hi + (size_t)tok * nb;
    bsl[ct] = xs_lo + (size_t)tok * nb;
  }
  v4f acc[2][2][kColTiles];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < kColTiles; ++ct) acc[m][rt][ct] = (v4f){0.f, 0.f, 0.f, 0.f};
  int kb = 0;
  for (; kb + 16 <= nb; kb += 16)
    mx_superstep<4, 2, 2>(kb, g, nct, arow, asrow, bh, bl, bsh, bsl, acc);
  for (; kb < nb; kb += 4) mx_superstep<1, 2, 2>(kb, g, nct, arow, asrow, bh, bl, bsh, bsl, acc);

  // epilogue: h = SiLU(g) * u, then the 2-term E4M3 split per 32 features.
  // The wave's 32 features nw0..nw0+31 form exactly one MX block; lane (r, g)
  // holds features 16 rt + 4 g + i for token column r.
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
    if (ct >= nct) continue;
    float h[2][4];
    float amax = 0.0f;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[rt][i] = silu_f32(acc[0][rt][ct][i]) * acc[1][rt][ct][i];
        amax = fmaxf(amax, fabsf(h[rt][i]));
      }
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    const uint32_t b1 = e4m3_block_scale_byte(amax);
    const float s1 = e8m0_to_f32(b1), s1inv = e8m0_to_f32(254u - b1);
    float hi[2][4], rs[2][4];
    float ramax = 0.0f;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[rt][i] = round_e4m3(h[rt][i] * s1inv);
        rs[rt][i] = h[rt][i] - hi[rt][i] * s1;
        ramax = fmaxf(ramax, fabsf(rs[rt][i]));
      }
    ramax = fmaxf(ramax, __shfl_xor(ramax, 16, 64));
    ramax = fmaxf(ramax, __shfl_xor(ramax, 32, 64));
    const uint32_t b2 = e4m3_block_scale_byte(ramax);
    const float s2inv = e8m0_to_f32(254u - b2);
    const int i = 16 * ct + r;
    if (i < ti.cnt) {
      const size_t pos = (size_t)ti.base + ti.row0 + i;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const size_t off = pos * f + nw0 + 16 * rt + 4 * g;
        *reinterpret_cast<uint32_t*>(hq_hi + off) = pack4_e4m3(hi[rt][0], hi[rt][1], hi[rt][2], hi[rt][3]);
        *reinterpret_cast<uint32_t*>(hq_lo + off) =
            pack4_e4m3(round_e4m3(rs[rt][0] * s2inv), round_e4m3(rs[rt][1] * s2inv),
                       round_e4m3(rs[rt][2] * s2inv), round_e4m3(rs[rt][3] * s2inv));
      }
      if (g == 0) {
        hs_hi[pos * nbf + (nw0 >> 5)] = (uint8_t)b1;
        hs_lo[pos * nbf + (nw0 >> 5)] = (uint8_t)b2;
      }
    }
  }
}

// ------------------------------------------------------------- down + combine
// grid: (max_tiles, d / 128), block 256. y[t, m] += gate[pair] * (Wd[e] h)[m]
// by fp32 atomic adds (y is cleared first).
__global__ __launch_bounds__(256) void gemm_down_kernel(
    int d, int f, const uint8_t* __restrict__ dq, const uint8_t* __restrict__ ds,
    const uint8_t* __restrict__ hq_hi, const uint8_t* __restrict__ hq_lo,
    const uint8_t* __restrict__ hs_hi, const uint8_t* __restrict__ hs_lo,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    const float* __restrict__ gate, int k, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, float* __restrict__ y) {
  TileInfo ti;
  if (!load_tile(tiles, ntiles, offsets, ti)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int nbf = f >> 5;
  const int nct = (ti.cnt + 15) >> 4;
  const int mw0 = blockIdx.y * kRowsPerBlock + wave * kRowsPerWave;
  const uint8_t* arow[1][2];
  const uint8_t* asrow[1][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const size_t row = (size_t)ti.e * d + mw0 + 16 * rt + r;
    arow[0][rt] = dq + row * (size_t)(f >> 1);
    asrow[0][rt] = ds + row * (size_t)nbf;
  }
  const uint8_t* bh[kColTiles];
  const uint8_t* bl[kColTiles];
  const uint8_t* bsh[kColTiles];
  const uint8_t* bsl[kColTiles];
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
    int i = 16 * ct + r;
    if (i >= ti.cnt) i = 0;
    const size_t pos = (size_t)ti.base + ti.row0 + i;
    bh[ct] = hq_hi + pos * f;
    bl[ct] = hq_lo + pos * f;
    bsh[ct] = hs_hi + pos * nbf;
    bsl[ct] = hs_lo + pos * nbf;
  }
  v4f acc[1][2][kColTiles];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) acc[0][rt][ct] = (v4f){0.f, 0.f, 0.f, 0.f};
  int kb = 0;
  for (; kb + 16 <= nbf; kb += 16)
    mx_superstep<4, 1, 2>(kb, g, nct, arow, asrow, bh, bl, bsh, bsl, acc);
  for (; kb < nbf; kb += 4) mx_superstep<1, 1, 2>(kb, g, nct, arow, asrow, bh, bl, bsh, bsl, acc);

  // epilogue: lane (r, g) holds rows mw0 + 16 rt + 4 g + i of token column r
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
    if (ct >= nct) continue;
    const int i = 16 * ct + r;
    if (i >= ti.cnt) continue;
    const int pair = perm[ti.base + ti.row0 + i];
    const int tok = pair / k;
    const float gw = gate[pair];
    float* yr = y + (size_t)tok * d + mw0 + 4 * g;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int q = 0; q < 4; ++q) atomicAdd(yr + 16 * rt + q, gw * acc[0][rt][ct][q]);
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float4* __restrict__ p, size_t n4) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

hipError_t launch_clear_y(float* y, int T, int d, hipStream_t st) {
  const size_t n4 = (size_t)T * d / 4;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)std::min<size_t>((n4 + 255) / 256, 4096)),
                     dim3(256), 0, st, reinterpret_cast<float4*>(y), n4);
  return hipGetLastError();
}

hipError_t launch_gemm_gateup(int T, const Shape& s, const ExpertWeights& w, const uint8_t* xq,
                              const uint8_t* xs, const int32_t* offsets, const int32_t* perm,
                              const int32_t* tiles, const int32_t* ntiles, int max_tiles,
                              uint8_t* hq, uint8_t* hs, hipStream_t st) {
  if (T <= 0 || max_tiles <= 0) return hipSuccess;
  const size_t P = (size_t)T * s.k;
  const size_t xplane = (size_t)T * s.d, xsplane = (size_t)T * (s.d / 32);
  const size_t hplane = P * s.f, hsplane = P * (s.f / 32);
  dim3 g1(max_tiles, s.f / kRowsPerBlock);
  hipLaunchKernelGGL(gemm_gateup_kernel, g1, dim3(256), 0, st, s.d, s.f, s.k, w.gate_q, w.gate_s,
                     w.up_q, w.up_s, xq, xq + xplane, xs, xs + xsplane, offsets, perm, tiles,
                     ntiles, hq, hq + hplane, hs, hs + hsplane);
  return hipGetLastError();
}

hipError_t launch_gemm_down(int T, const Shape& s, const ExpertWeights& w, const float* gate,
                            const int32_t* offsets, const int32_t* perm, const int32_t* tiles,
                            const int32_t* ntiles, int max_tiles, const uint8_t* hq,
                            const uint8_t* hs, float* y, hipStream_t st) {
  if (T <= 0 || max_tiles <= 0) return hipSuccess;
  const size_t P = (size_t)T * s.k;
  const size_t hplane = P * s.f, hsplane = P * (s.f / 32);
  dim3 g2(max_tiles, s.d / kRowsPerBlock);
  hipLaunchKernelGGL(gemm_down_kernel, g2, dim3(256), 0, st, s.d, s.f, w.down_q, w.down_s, hq,
                     hq + hplane, hs, hs + hsplane, offsets, perm, gate, s.k, tiles, ntiles, y);
  return hipGetLastError();
}

}  // namespace k3
