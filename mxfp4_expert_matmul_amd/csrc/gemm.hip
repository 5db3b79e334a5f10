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
// One workgroup = 4 waves = one (tile, row block): up to kTileM = 64 tokens
// of one expert (a tile of the grouped pairs) times a block of weight rows.
//   gate/up (kGateUp): 128 features = 128 gate rows + the same 128 up rows;
//   down    (kDown):   256 output rows.
// Wave w owns 32 features (gate/up: two 16-row MFMA tiles of gate and the
// same two of up, so SwiGLU pairs sit in one lane) or 64 rows (down: four
// 16-row tiles), for all 64 tokens of the tile (four 16-column MFMA tiles).
// Two workgroups share a CU, so one computes while the other waits for
// memory.
//
// Weights (tiled layout, layout.hip) go straight to registers: one MFMA A
// operand is one 1 KB tile, read with one coalesced 16-byte-per-lane load,
// one chunk ahead of the MFMAs; a scale dword per lane covers 4 K tiles.
// Activations (two E4M3 terms + scales) of the tile's tokens are copied once
// per workgroup straight into LDS (global_load_lds, four 256-byte token rows
// per wave instruction; piece p of token row t at slot p ^ (t % 16) so an
// MFMA column group reads 16 distinct bank groups), double-buffered.
// K is walked in chunks of two 128-column tiles (a last chunk of one tile
// when K/128 is odd); MFMA step s of chunk c is K tile 2c + s, and MFMA
// slot-block kappa is that tile's 32-column block kappa.
constexpr int kGateUp = 0;
constexpr int kDown = 1;
constexpr int kChunkTiles = 2;                  // K tiles (128 columns) per chunk
constexpr int kActRow = kChunkTiles * 128;      // LDS bytes per token row and term
constexpr int kScRow = kChunkTiles * 4;         // LDS scale bytes per token row and term
constexpr int kThreads = 256;

template <int MODE>
struct GemmShape {
  static constexpr int NM = (MODE == kGateUp) ? 2 : 1;   // weight matrices
  static constexpr int NRT = (MODE == kGateUp) ? 2 : 4;  // 16-row tiles per matrix per wave
  static constexpr int kRowsPerWave = NRT * 16;           // output rows (features) per wave
  static constexpr int kRowsPerBlock = 4 * kRowsPerWave;  // output rows per workgroup
};

struct TileInfo {
  int e, row0, cnt, base;  // expert, first row within the expert, tokens, offsets[e]
};

// Workgroup -> (tile, row block). Workgroups are dispatched round-robin over
// the 8 XCDs. Each XCD takes a contiguous range of the tile list (the tiles
// of one expert are adjacent in it) and walks it tile by tile, all row blocks
// of a tile back to back: a tile's activations are fetched into that XCD's
// L2 once, and consecutive tiles of one expert find its weights in the
// XCD's L2 or the memory-side cache. (Interleaving the row blocks of two
// tiles measured slower.)
__device__ __forceinline__ void block_coords(int nrb, int ntiles, int& tile, int& rb) {
  const int lid = blockIdx.x;
  const int xcd = lid & 7, q = lid >> 3;
  const int tpx = (ntiles + 7) / 8;  // tiles per XCD
  const int lt = q / nrb;            // tile within the XCD's range
  rb = q % nrb;
  tile = (lt < tpx) ? xcd * tpx + lt : ntiles;  // ntiles = no work
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

struct ActLds {
  uint8_t a[2][kTileM][kActRow];  // activation terms, swizzled
  uint8_t s[2][kTileM][kScRow];   // activation scales (E8M0), per 32-column block
};

template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void mx_gemm_kernel(
    int K, int nrows, int f_out, int k, const uint8_t* __restrict__ wq0,
    const uint8_t* __restrict__ ws0, const uint8_t* __restrict__ wq1,
    const uint8_t* __restrict__ ws1, const uint8_t* __restrict__ act_hi,
    const uint8_t* __restrict__ act_lo, const uint8_t* __restrict__ acts_hi,
    const uint8_t* __restrict__ acts_lo, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, int nrb, uint8_t* __restrict__ out_hi,
    uint8_t* __restrict__ out_lo, uint8_t* __restrict__ outs_hi, uint8_t* __restrict__ outs_lo,
    float* __restrict__ slots) {
  using G = GemmShape<MODE>;
  constexpr int NM = G::NM, NRT = G::NRT;
  constexpr int NCT = 4;  // 16-token MFMA column tiles per wave
  // two separately named buffers (not an array indexed by a runtime number)
  // so reads of one need not wait for the direct-to-LDS loads filling the other
  __shared__ __attribute__((aligned(16))) ActLds lds0;
  __shared__ __attribute__((aligned(16))) ActLds lds1;
  __shared__ int tok_lds[kTileM];

  int tile, rb;
  block_coords(nrb, ntiles[0], tile, rb);
  TileInfo ti;
  if (!load_tile(tile, tiles, ntiles, offsets, ti)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nw = wave;
  const int r = lane & 15, g = lane >> 4;
  const int nb = K >> 5, KT = K >> 7, KG = (KT + 3) >> 2, RT = nrows >> 4;
  const int row_base = rb * G::kRowsPerBlock;          // first output row of the block
  const int w0 = row_base + nw * G::kRowsPerWave;       // first output row of this wave
  const int m0 = 0;                                     // first tile token of this wave
  const int nct = max(0, min(NCT, (ti.cnt - m0 + 15) >> 4));  // token tiles of this wave
  const bool wave_on = (w0 < nrows) && (nct > 0);

  // activation row (token for gate/up, sorted pair position for down) per tile row
  if (tid < kTileM) {
    const int i = (tid < ti.cnt) ? tid : 0;
    tok_lds[tid] = (MODE == kGateUp) ? perm[ti.base + ti.row0 + i] / k : ti.base + ti.row0 + i;
  }
  __syncthreads();

  // ---- weights: tile (rt, kt) of matrix m at wq[m] + ((e RT + rt) KT + kt) 1024 + 16 lane
  const int rt0 = (wave_on ? w0 : 0) >> 4;  // first row tile of this wave
  const uint8_t* wq_t[NM];
  const uint32_t* ws_t[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const uint8_t* q = (m == 0) ? wq0 : wq1;
    const uint8_t* sc = (m == 0) ? ws0 : ws1;
    wq_t[m] = q + (((size_t)ti.e * RT + rt0) * KT) * 1024 + 16 * lane;
    ws_t[m] = reinterpret_cast<const uint32_t*>(sc + (((size_t)ti.e * RT + rt0) * KG) * 256) + lane;
  }
  struct WStage {
    uint4 q[NM][NRT][kChunkTiles];
  };
  auto w_load = [&](int c, int S, WStage& ws) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int s = 0; s < kChunkTiles; ++s)
          if (s < S)
            ws.q[m][rt][s] = *reinterpret_cast<const uint4*>(
                wq_t[m] + ((size_t)rt * KT + kChunkTiles * c + s) * 1024);
  };
  // scale dwords of the current group of 4 K tiles (sw) and of the next
  // (swn), loaded one iteration ahead so the MFMAs never wait on a load that
  // was issued behind direct-to-LDS copies
  int sw[NM][NRT], swn[NM][NRT];
  auto s_load = [&](int kg, int (&dst)[NM][NRT]) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) dst[m][rt] = (int)ws_t[m][((size_t)rt * KG + kg) * 64];
  };

  // ---- activations: wave instruction j = 8 wave + i (32 per chunk): term
  // j / 16, token rows 4 (j % 16) .. +3; lane -> row + lane / 16, slot lane % 16
  // holding piece slot ^ (row % 16). Scales: one 4-byte copy per lane, wave w
  // -> term w / 2, rows 32 (w % 2) + lane / 2, half lane % 2.
  const uint8_t* act_t = (wave < 2) ? act_hi : act_lo;
  uint32_t asrc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = 8 * wave + i;
    const int row = 4 * (j & 15) + (lane >> 4);
    asrc[i] = (uint32_t)tok_lds[row] * (uint32_t)K + 16u * (uint32_t)((lane & 15) ^ (row & 15));
  }
  const int sc_row = 32 * (wave & 1) + (lane >> 1);
  const uint8_t* sc_src = ((wave < 2) ? acts_hi : acts_lo) + (size_t)tok_lds[sc_row] * nb;
  auto act_issue = [&](ActLds& L, int c, int S) {
    const uint32_t kb = (uint32_t)(kChunkTiles * c) * 128u;  // first column of the chunk
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 8 * wave + i;
      const int term = j >> 4, row0 = 4 * (j & 15);
      if (row0 < ti.cnt) {
        uint32_t off = asrc[i] + kb;
        if (S < kChunkTiles) off -= 16u * (((lane & 15) ^ ((row0 + (lane >> 4)) & 15)) & 8u);
        __builtin_amdgcn_global_load_lds(act_t + off, (lds_ptr)&L.a[term][row0][0], 16, 0, 0);
      }
    }
    {
      const int half = (S < kChunkTiles) ? 0 : (lane & 1);
      __builtin_amdgcn_global_load_lds(sc_src + (kb >> 5) + 4 * half,
                                       (lds_ptr)&L.s[wave >> 1][32 * (wave & 1)][0], 4, 0, 0);
    }
  };

  v4f acc[NM][NRT][NCT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[m][rt][ct] = (v4f){0.f, 0.f, 0.f, 0.f};

  // one chunk of MFMAs; SEL = byte of the scale dwords for step 0 (0 or 2)
  auto compute = [&](const ActLds& L, int S, const WStage& ws, int sel) {
#pragma unroll
    for (int s = 0; s < kChunkTiles; ++s) {
      if (s >= S) break;
      // pieces of slot-blocks g/2 and 2 + g/2 of tile s (token row % 16 == r)
      const int c0 = 16 * ((8 * s + g) ^ r);
      const int c1 = 16 * ((8 * s + 4 + g) ^ r);
      const int sb = 4 * s + g;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        if (ct < nct) {
          const int tr = m0 + 16 * ct + r;
          const v8i bh = fp8_operand(*reinterpret_cast<const uint4*>(&L.a[0][tr][c0]),
                                     *reinterpret_cast<const uint4*>(&L.a[0][tr][c1]));
          const v8i bl = fp8_operand(*reinterpret_cast<const uint4*>(&L.a[1][tr][c0]),
                                     *reinterpret_cast<const uint4*>(&L.a[1][tr][c1]));
          const int sh = L.s[0][tr][sb];
          const int sl = L.s[1][tr][sb];
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
              const v8i a = fp4_operand(ws.q[m][rt][s]);
              // scale byte (sel + s) of the A scale dword
              if (sel + s == 0) {
                acc[m][rt][ct] = mfma_fp4_fp8<0>(a, sw[m][rt], bh, sh, acc[m][rt][ct]);
                acc[m][rt][ct] = mfma_fp4_fp8<0>(a, sw[m][rt], bl, sl, acc[m][rt][ct]);
              } else if (sel + s == 1) {
                acc[m][rt][ct] = mfma_fp4_fp8<1>(a, sw[m][rt], bh, sh, acc[m][rt][ct]);
                acc[m][rt][ct] = mfma_fp4_fp8<1>(a, sw[m][rt], bl, sl, acc[m][rt][ct]);
              } else if (sel + s == 2) {
                acc[m][rt][ct] = mfma_fp4_fp8<2>(a, sw[m][rt], bh, sh, acc[m][rt][ct]);
                acc[m][rt][ct] = mfma_fp4_fp8<2>(a, sw[m][rt], bl, sl, acc[m][rt][ct]);
              } else {
                acc[m][rt][ct] = mfma_fp4_fp8<3>(a, sw[m][rt], bh, sh, acc[m][rt][ct]);
                acc[m][rt][ct] = mfma_fp4_fp8<3>(a, sw[m][rt], bl, sl, acc[m][rt][ct]);
              }
            }
        }
        // keep one column tile's B fragments live at a time
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // K loop, two chunks (= one scale group of 4 K tiles) per iteration so each
  // LDS buffer and each scale byte is named statically.
  const int nchunks = (KT + kChunkTiles - 1) / kChunkTiles;
  auto tiles_of = [&](int c) { return min(kChunkTiles, KT - kChunkTiles * c); };
  WStage wa, wb;
  act_issue(lds0, 0, tiles_of(0));
  if (wave_on) {
    w_load(0, tiles_of(0), wa);
    s_load(0, sw);
  }
  __syncthreads();  // also waits for this thread's direct-to-LDS loads
  for (int c = 0; c < nchunks; c += 2) {
    {  // even chunk c: buffer 0, weights wa, scale bytes 0/1
      const bool more = (c + 1) < nchunks;
      if (more) {
        act_issue(lds1, c + 1, tiles_of(c + 1));
        if (wave_on) w_load(c + 1, tiles_of(c + 1), wb);
      }
      if (wave_on) compute(lds0, tiles_of(c), wa, 0);
      __syncthreads();
      if (!more) break;
    }
    {  // odd chunk c + 1: buffer 1, weights wb, scale bytes 2/3
      const bool more = (c + 2) < nchunks;
      if (more) {
        act_issue(lds0, c + 2, tiles_of(c + 2));
        if (wave_on) {
          w_load(c + 2, tiles_of(c + 2), wa);
          s_load((c + 2) >> 1, swn);
        }
      }
      if (wave_on) compute(lds1, tiles_of(c + 1), wb, 2);
      __syncthreads();
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) sw[m][rt] = swn[m][rt];
    }
  }
  if (!wave_on) return;

  if (MODE == kGateUp) {
    // h = SiLU(g) * u, split into two E4M3 terms per 32 features (the wave's
    // 32 features are one MX block; lane (r, g) holds features 16 rt + 4 g + i
    // of token column r).
    const int nbf = f_out >> 5;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
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
      const int i = m0 + 16 * ct + r;
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
    // this pair's expert output, rows w0 + 16 rt + 4 g + q of token column r,
    // stored in the pair's own slot (no atomics; summed per token later)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if (ct >= nct) continue;
      const int i = m0 + 16 * ct + r;
      if (i >= ti.cnt) continue;
      const int pair = perm[ti.base + ti.row0 + i];
      float* o = slots + (size_t)pair * nrows + w0 + 4 * g;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
        *reinterpret_cast<float4*>(o + 16 * rt) =
            make_float4(acc[0][rt][ct][0], acc[0][rt][ct][1], acc[0][rt][ct][2], acc[0][rt][ct][3]);
    }
  }
}

// y[t] = sum_j gate[t,j] * slot[t*k + j], j in order; pairs whose expert is
// outside [0, E) contribute zero. One thread per 4 outputs.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ slots,
                                                      const int32_t* __restrict__ idx,
                                                      const float* __restrict__ gate, int T,
                                                      int d, int k, int E, float* __restrict__ y) {
  const int d4 = d >> 2;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)T * d4) return;
  const int t = (int)(i / d4), c = (int)(i % d4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int e = idx[(size_t)t * k + j];
    if (e < 0 || e >= E) continue;
    const float gw = gate[(size_t)t * k + j];
    const float4 v = reinterpret_cast<const float4*>(slots + ((size_t)t * k + j) * d)[c];
    acc.x = fmaf(gw, v.x, acc.x);
    acc.y = fmaf(gw, v.y, acc.y);
    acc.z = fmaf(gw, v.z, acc.z);
    acc.w = fmaf(gw, v.w, acc.w);
  }
  reinterpret_cast<float4*>(y)[i] = acc;
}

// 8 XCDs x tiles per XCD x row blocks; the kernel sees the actual tile count
// and idles workgroups beyond it
static unsigned gemm_grid(int max_tiles, int nrb) {
  return (unsigned)(8 * ((max_tiles + 7) / 8) * nrb);
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
  hipLaunchKernelGGL(mx_gemm_kernel<kGateUp>, dim3(gemm_grid(max_tiles, nrb)), dim3(kThreads), 0,
                     st, s.d, s.f, s.f, s.k, w.gate_q, w.gate_s, w.up_q, w.up_s, xq, xq + xplane,
                     xs, xs + xsplane, offsets, perm, tiles, ntiles, nrb, hq, hq + hplane, hs,
                     hs + hsplane, nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm_down(int T, const Shape& s, const ExpertWeights& w, const int32_t* offsets,
                            const int32_t* perm, const int32_t* tiles, const int32_t* ntiles,
                            int max_tiles, const uint8_t* hq, const uint8_t* hs, float* slots,
                            hipStream_t st) {
  if (T <= 0 || max_tiles <= 0) return hipSuccess;
  const size_t P = (size_t)T * s.k;
  const size_t hplane = P * s.f, hsplane = P * (s.f / 32);
  constexpr int rpb = GemmShape<kDown>::kRowsPerBlock;
  const int nrb = (s.d + rpb - 1) / rpb;
  hipLaunchKernelGGL(mx_gemm_kernel<kDown>, dim3(gemm_grid(max_tiles, nrb)), dim3(kThreads), 0,
                     st, s.f, s.d, s.f, s.k, w.down_q, w.down_s, nullptr, nullptr, hq, hq + hplane,
                     hs, hs + hsplane, offsets, perm, tiles, ntiles, nrb, nullptr, nullptr, nullptr,
                     nullptr, slots);
  return hipGetLastError();
}

hipError_t launch_combine(const float* slots, const int32_t* idx, const float* gate, int T,
                          const Shape& s, float* y, hipStream_t st) {
  const size_t n = (size_t)T * (s.d / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, slots,
                     idx, gate, T, s.d, s.k, s.E, y);
  return hipGetLastError();
}

}  // namespace k3
