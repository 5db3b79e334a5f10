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

// sa: the A scale register, OPSEL_A picks its byte; sb: the B scale in byte 0
template <int OPSEL_A>
__device__ __forceinline__ v4f mfma_fp4_fp8(v8i a, int sa, v8i b, int sb, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kFmtFp4, kFmtFp8, OPSEL_A, sa,
                                                         0, sb);
}

// ------------------------------------------------------------- grouped GEMM
// One workgroup = 4 waves = one (tile, row block): up to kTileM tokens of one
// expert (a tile of the grouped pairs) times kRowsPerBlock weight rows.
//   gate/up (kMode = kGateUp): each wave owns 32 features, i.e. two 16-row
//     MFMA tiles of the gate matrix and the same two of the up matrix, so
//     SwiGLU pairs sit in the same lanes; a block covers 128 features.
//   down (kMode = kDown): each wave owns 64 output rows (four 16-row tiles);
//     a block covers 256 rows.
// The K dimension is walked in chunks of 8 MX blocks (256 elements; a last
// chunk of 4 blocks when K/32 is not a multiple of 8). Per chunk:
//   * activations (two E4M3 terms) of the tile's tokens are copied once per
//     workgroup straight from global memory into LDS (global_load_lds, 16
//     bytes per lane, four 256-byte token rows per wave instruction) and read
//     by every wave as MFMA B operands; double-buffered. Within a token row
//     the 16-byte piece p is stored at slot p ^ (row % 16), so the 16 lanes
//     of an MFMA column group (16 consecutive rows, same piece) read 16
//     distinct bank groups; the scales go through registers;
//   * each wave's weight rows are loaded straight into registers one chunk
//     ahead (two contiguous MX blocks per lane, 128 contiguous bytes per row).
// Physical block of MFMA slot-block kappa at step s of a chunk with S steps
// = chunk base + S*kappa + s.
constexpr int kGateUp = 0;
constexpr int kDown = 1;
constexpr int kChunkBlocks = 8;                 // MX blocks per K chunk
constexpr int kActRow = kChunkBlocks * 32;      // LDS bytes per token row and term
constexpr int kColTiles = kTileM / 16;

template <int MODE>
struct GemmShape {
  static constexpr int NM = (MODE == kGateUp) ? 2 : 1;   // weight matrices
  static constexpr int NRT = (MODE == kGateUp) ? 2 : 4;  // 16-row tiles per matrix per wave
  static constexpr int kRowsPerWave = NM * NRT * 16 / NM;  // output rows per wave (per matrix)
  static constexpr int kRowsPerBlock = 4 * kRowsPerWave;
};

struct TileInfo {
  int e, row0, cnt, base;  // expert, first row within the expert, tokens, offsets[e]
};

// Workgroup -> (tile, row block). Workgroups are dispatched round-robin over
// the 8 XCDs; consecutive workgroups of one XCD take consecutive row blocks
// of the same tile, so a tile's activations are fetched into that XCD's L2
// once and its row blocks run together.
__device__ __forceinline__ void block_coords(int nrb, int& tile, int& rb) {
  const int lid = blockIdx.x;
  const int xcd = lid & 7, q = lid >> 3;
  tile = (q / nrb) * 8 + xcd;
  rb = q % nrb;
}

__device__ __forceinline__ bool load_tile(int tile, const int32_t* tiles, const int32_t* ntiles,
                                          const int32_t* offsets, TileInfo& ti) {
  if (tile >= ntiles[0]) return false;
  ti.e = tiles[2 * tile];
  ti.row0 = tiles[2 * tile + 1];
  ti.base = offsets[ti.e];
  const int total = offsets[ti.e + 1] - ti.base;
  ti.cnt = min(total - ti.row0, kTileM);
  return ti.cnt > 0;
}

typedef __attribute__((address_space(3))) void* lds_ptr;

template <int MODE>
__global__ __launch_bounds__(256, 2) void mx_gemm_kernel(
    int K, int nrows, int f_out, int k, const uint8_t* __restrict__ wq0,
    const uint8_t* __restrict__ ws0, const uint8_t* __restrict__ wq1,
    const uint8_t* __restrict__ ws1, const uint8_t* __restrict__ act_hi,
    const uint8_t* __restrict__ act_lo, const uint8_t* __restrict__ acts_hi,
    const uint8_t* __restrict__ acts_lo, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, int nrb, uint8_t* __restrict__ out_hi,
    uint8_t* __restrict__ out_lo, uint8_t* __restrict__ outs_hi, uint8_t* __restrict__ outs_lo,
    const float* __restrict__ gate, float* __restrict__ y) {
  using G = GemmShape<MODE>;
  constexpr int NM = G::NM, NRT = G::NRT;
  __shared__ __attribute__((aligned(16))) uint8_t act_lds[2][2][kTileM][kActRow];
  __shared__ __attribute__((aligned(16))) uint8_t sc_lds[2][2][kTileM][kChunkBlocks];
  __shared__ int tok_lds[kTileM];

  int tile, rb;
  block_coords(nrb, tile, rb);
  TileInfo ti;
  if (!load_tile(tile, tiles, ntiles, offsets, ti)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int nb = K >> 5;
  const int nct = (ti.cnt + 15) >> 4;
  const int w0 = rb * G::kRowsPerBlock + wave * G::kRowsPerWave;  // first row of this wave
  const bool wave_on = w0 < nrows;

  // activation row (token for gate/up, sorted pair position for down) per tile row
  if (tid < kTileM) {
    const int i = (tid < ti.cnt) ? tid : 0;
    tok_lds[tid] = (MODE == kGateUp) ? perm[ti.base + ti.row0 + i] / k : ti.base + ti.row0 + i;
  }
  __syncthreads();

  // weight addressing: uniform per-expert bases + one 32-bit lane offset
  // (rows clamped into range for waves past the end)
  const size_t qstride = (size_t)(K >> 1);
  const uint8_t* wqb[NM];
  const uint8_t* wsb[NM];
  wqb[0] = wq0 + (size_t)ti.e * nrows * qstride;
  wsb[0] = ws0 + (size_t)ti.e * nrows * nb;
  if (NM == 2) {
    wqb[NM - 1] = wq1 + (size_t)ti.e * nrows * qstride;
    wsb[NM - 1] = ws1 + (size_t)ti.e * nrows * nb;
  }
  const int row_l = (wave_on ? w0 : 0) + r;
  const uint32_t qoff = (uint32_t)row_l * (uint32_t)(K >> 1);
  const uint32_t soff = (uint32_t)row_l * (uint32_t)nb;

  // activations of one chunk straight into LDS: wave instruction I (8 per
  // wave) moves term I / 16, rows 4 (I % 16) .. +3, lane l -> row + l / 16,
  // slot l % 16 holding piece (l % 16) ^ (row % 16). Row groups past the
  // tile's tokens are skipped; pieces past a 4-block tail chunk re-read
  // pieces of the chunk (their slots are never read).
  auto act_issue = [&](int buf, int kb0, int cblocks) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int I = wave * 8 + i;
      const int term = I >> 4, row0 = 4 * (I & 15);
      if (row0 < ti.cnt) {
        const int row = row0 + (lane >> 4);
        int piece = (lane & 15) ^ (row & 15);
        if (cblocks < kChunkBlocks) piece &= 2 * cblocks - 1;
        const uint8_t* src =
            (term ? act_lo : act_hi) + (size_t)tok_lds[row] * K + 32 * kb0 + 16 * piece;
        __builtin_amdgcn_global_load_lds(src, (lds_ptr)&act_lds[buf][term][row0][0], 16, 0, 0);
      }
    }
  };
  auto sc_load = [&](int kb0, int cblocks) {
    uint2 v = make_uint2(0u, 0u);
    if (tid < 2 * kTileM) {
      const int term = tid >> 6, tk = tid & 63;
      if (tk < ti.cnt) {
        const uint8_t* src = (term ? acts_lo : acts_hi) + (size_t)tok_lds[tk] * nb + kb0;
        if (cblocks == kChunkBlocks)
          v = *reinterpret_cast<const uint2*>(src);
        else
          v.x = *reinterpret_cast<const uint32_t*>(src);
      }
    }
    return v;
  };
  auto sc_store = [&](int buf, uint2 v) {
    if (tid < 2 * kTileM) *reinterpret_cast<uint2*>(&sc_lds[buf][tid >> 6][tid & 63][0]) = v;
  };

  // weights of one chunk: S contiguous blocks per lane per row tile
  struct WStage {
    uint4 q[NM][NRT][2];
    int s[NM][NRT];
  };
  auto w_load = [&](int kb0, int S, WStage& ws) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const uint8_t* p = wqb[m] + 16 * rt * qstride + qoff + 16 * (kb0 + S * g);
        const uint8_t* ps = wsb[m] + 16 * rt * nb + soff + kb0 + S * g;
        ws.q[m][rt][0] = *reinterpret_cast<const uint4*>(p);
        if (S == 2) {
          ws.q[m][rt][1] = *reinterpret_cast<const uint4*>(p + 16);
          ws.s[m][rt] = *reinterpret_cast<const uint16_t*>(ps);
        } else {
          ws.s[m][rt] = *ps;
        }
      }
  };

  v4f acc[NM][NRT][kColTiles];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < kColTiles; ++ct) acc[m][rt][ct] = (v4f){0.f, 0.f, 0.f, 0.f};

  // one chunk of MFMAs from LDS buffer `buf` with weights `ws`
  auto compute = [&](int buf, int S, const WStage& ws) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s >= S) break;
      // pieces of slot-blocks g/2 and 2 + g/2, swizzled by the row (row % 16 == r)
      const int c0 = 16 * ((2 * (S * (g >> 1) + s) + (g & 1)) ^ r);
      const int c1 = 16 * ((2 * (S * (2 + (g >> 1)) + s) + (g & 1)) ^ r);
      const int sb = S * g + s;  // scale block of this lane
#pragma unroll
      for (int ct = 0; ct < kColTiles; ++ct) {
        if (ct < nct) {
          const int tr = 16 * ct + r;
          const v8i bh = fp8_operand(*reinterpret_cast<const uint4*>(&act_lds[buf][0][tr][c0]),
                                     *reinterpret_cast<const uint4*>(&act_lds[buf][0][tr][c1]));
          const v8i bl = fp8_operand(*reinterpret_cast<const uint4*>(&act_lds[buf][1][tr][c0]),
                                     *reinterpret_cast<const uint4*>(&act_lds[buf][1][tr][c1]));
          const int sh = sc_lds[buf][0][tr][sb];
          const int sl = sc_lds[buf][1][tr][sb];
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
              const v8i a = fp4_operand(ws.q[m][rt][s]);
              if (s == 0) {
                acc[m][rt][ct] = mfma_fp4_fp8<0>(a, ws.s[m][rt], bh, sh, acc[m][rt][ct]);
                acc[m][rt][ct] = mfma_fp4_fp8<0>(a, ws.s[m][rt], bl, sl, acc[m][rt][ct]);
              } else {
                acc[m][rt][ct] = mfma_fp4_fp8<1>(a, ws.s[m][rt], bh, sh, acc[m][rt][ct]);
                acc[m][rt][ct] = mfma_fp4_fp8<1>(a, ws.s[m][rt], bl, sl, acc[m][rt][ct]);
              }
            }
        }
      }
    }
  };

  const int nfull = nb / kChunkBlocks;
  const bool tail = (nb % kChunkBlocks) != 0;  // one last chunk of 4 blocks
  const int nchunks = nfull + (tail ? 1 : 0);
  WStage wcur, wnxt;
  {
    const int cb = (nfull > 0) ? kChunkBlocks : 4;
    act_issue(0, 0, cb);
    w_load(0, cb / 4, wcur);
    sc_store(0, sc_load(0, cb));
  }
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int S = (c < nfull) ? 2 : 1;
    const bool more = (c + 1) < nchunks;
    const int cb_next = ((c + 1) < nfull) ? kChunkBlocks : 4;
    uint2 scn = make_uint2(0u, 0u);
    if (more) {
      act_issue((c + 1) & 1, (c + 1) * kChunkBlocks, cb_next);
      w_load((c + 1) * kChunkBlocks, cb_next / 4, wnxt);
      scn = sc_load((c + 1) * kChunkBlocks, cb_next);
    }
    if (wave_on) compute(c & 1, S, wcur);
    if (more) sc_store((c + 1) & 1, scn);
    __syncthreads();  // also waits for this thread's direct-to-LDS loads
    wcur = wnxt;
  }
  if (!wave_on) return;

  if (MODE == kGateUp) {
    // h = SiLU(g) * u, split into two E4M3 terms per 32 features (the wave's
    // 32 features are one MX block; lane (r, g) holds features 16 rt + 4 g + i
    // of token column r).
    const int nbf = f_out >> 5;
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) {
      if (ct >= nct) continue;
      float h[2][4];
      float amax = 0.0f;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[rt][i] = silu_f32(acc[0][rt][ct][i]) * acc[NM - 1][rt][ct][i];
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
          const size_t off = pos * f_out + w0 + 16 * rt + 4 * g;
          *reinterpret_cast<uint32_t*>(out_hi + off) =
              pack4_e4m3(hi[rt][0], hi[rt][1], hi[rt][2], hi[rt][3]);
          *reinterpret_cast<uint32_t*>(out_lo + off) =
              pack4_e4m3(round_e4m3(rs[rt][0] * s2inv), round_e4m3(rs[rt][1] * s2inv),
                         round_e4m3(rs[rt][2] * s2inv), round_e4m3(rs[rt][3] * s2inv));
        }
        if (g == 0) {
          outs_hi[pos * nbf + (w0 >> 5)] = (uint8_t)b1;
          outs_lo[pos * nbf + (w0 >> 5)] = (uint8_t)b2;
        }
      }
    }
  } else {
    // y[t, m] += gate[pair] * acc: lane (r, g) holds rows w0 + 16 rt + 4 g + q
    // of token column r.
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) {
      if (ct >= nct) continue;
      const int i = 16 * ct + r;
      if (i >= ti.cnt) continue;
      const int pair = perm[ti.base + ti.row0 + i];
      const int tok = pair / k;
      const float gw = gate[pair];
      float* yr = y + (size_t)tok * nrows + w0 + 4 * g;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int q = 0; q < 4; ++q) atomicAdd(yr + 16 * rt + q, gw * acc[0][rt][ct][q]);
    }
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

static unsigned gemm_grid(int max_tiles, int nrb) {
  return (unsigned)(((max_tiles + 7) / 8) * 8 * nrb);
}

hipError_t launch_gemm_gateup(int T, const Shape& s, const ExpertWeights& w, const uint8_t* xq,
                              const uint8_t* xs, const int32_t* offsets, const int32_t* perm,
                              const int32_t* tiles, const int32_t* ntiles, int max_tiles,
                              uint8_t* hq, uint8_t* hs, hipStream_t st) {
  if (T <= 0 || max_tiles <= 0) return hipSuccess;
  const size_t P = (size_t)T * s.k;
  const size_t xplane = (size_t)T * s.d, xsplane = (size_t)T * (s.d / 32);
  const size_t hplane = P * s.f, hsplane = P * (s.f / 32);
  const int nrb = s.f / GemmShape<kGateUp>::kRowsPerBlock;
  hipLaunchKernelGGL(mx_gemm_kernel<kGateUp>, dim3(gemm_grid(max_tiles, nrb)), dim3(256), 0, st,
                     s.d, s.f, s.f, s.k, w.gate_q, w.gate_s, w.up_q, w.up_s, xq, xq + xplane, xs,
                     xs + xsplane, offsets, perm, tiles, ntiles, nrb, hq, hq + hplane, hs,
                     hs + hsplane, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm_down(int T, const Shape& s, const ExpertWeights& w, const float* gate,
                            const int32_t* offsets, const int32_t* perm, const int32_t* tiles,
                            const int32_t* ntiles, int max_tiles, const uint8_t* hq,
                            const uint8_t* hs, float* y, hipStream_t st) {
  if (T <= 0 || max_tiles <= 0) return hipSuccess;
  const size_t P = (size_t)T * s.k;
  const size_t hplane = P * s.f, hsplane = P * (s.f / 32);
  constexpr int rpb = GemmShape<kDown>::kRowsPerBlock;
  const int nrb = (s.d + rpb - 1) / rpb;
  hipLaunchKernelGGL(mx_gemm_kernel<kDown>, dim3(gemm_grid(max_tiles, nrb)), dim3(256), 0, st,
                     s.f, s.d, s.f, s.k, w.down_q, w.down_s, nullptr, nullptr, hq, hq + hplane, hs,
                     hs + hsplane, offsets, perm, tiles, ntiles, nrb, nullptr, nullptr, nullptr,
                     nullptr, gate, y);
  return hipGetLastError();
}

}  // namespace k3
