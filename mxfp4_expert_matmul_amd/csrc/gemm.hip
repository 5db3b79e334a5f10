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
// One MFMA step covers one 128-column K tile: the weight lane (r, g) holds
// the tile's 32-column block g of row r, and the activation lane (r, g) the
// 16-column pieces g and 4 + g of token r, so every K slot pairs the same
// physical column on both sides.
#include <type_traits>

#include "k3_device.h"
#include "k3_kernels.h"

namespace k3 {

constexpr int kFmtFp8 = 0;
constexpr int kFmtFp4 = 4;
constexpr int kNonTemporal = 2;  // buffer-load cache policy: streamed (nt)

// ------------------------------------------------------------- split of x
// Four threads per 32-element block of x, eight elements each: one 16-byte
// load, the block max over the four lanes by two shuffles, one 8-byte store
// per term, and the scale bytes from the block's first lane.
__global__ __launch_bounds__(256) void quant_x_kernel(const uint16_t* __restrict__ x, int nq,
                                                      uint8_t* __restrict__ xq_hi,
                                                      uint8_t* __restrict__ xq_lo,
                                                      uint8_t* __restrict__ xs_hi,
                                                      uint8_t* __restrict__ xs_lo) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // eighth-block index
  const bool on = i < nq;                         // every lane takes part in the shuffles
  float v[8];
  {
    const uint4 w = on ? reinterpret_cast<const uint4*>(x)[i] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_bits_to_f32(ww[j] & 0xffffu);
      v[2 * j + 1] = bf16_bits_to_f32(ww[j] >> 16);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const uint32_t b1 = e4m3_block_scale_byte(amax);
  const float s1 = e8m0_to_f32(b1), s1inv = e8m0_to_f32(254u - b1);
  float hi[8], r[8];
  float ramax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    hi[j] = round_e4m3(v[j] * s1inv);
    r[j] = v[j] - hi[j] * s1;
    ramax = fmaxf(ramax, fabsf(r[j]));
  }
  ramax = fmaxf(ramax, __shfl_xor(ramax, 1, 64));
  ramax = fmaxf(ramax, __shfl_xor(ramax, 2, 64));
  const uint32_t b2 = e4m3_block_scale_byte(ramax);
  const float s2inv = e8m0_to_f32(254u - b2);
  if (!on) return;
  reinterpret_cast<uint2*>(xq_hi)[i] =
      make_uint2(pack4_e4m3(hi[0], hi[1], hi[2], hi[3]), pack4_e4m3(hi[4], hi[5], hi[6], hi[7]));
  reinterpret_cast<uint2*>(xq_lo)[i] =
      make_uint2(pack4_e4m3(round_e4m3(r[0] * s2inv), round_e4m3(r[1] * s2inv),
                            round_e4m3(r[2] * s2inv), round_e4m3(r[3] * s2inv)),
                 pack4_e4m3(round_e4m3(r[4] * s2inv), round_e4m3(r[5] * s2inv),
                            round_e4m3(r[6] * s2inv), round_e4m3(r[7] * s2inv)));
  if ((i & 3) == 0) {
    xs_hi[i >> 2] = (uint8_t)b1;
    xs_lo[i >> 2] = (uint8_t)b2;
  }
}

hipError_t launch_quant_x(const uint16_t* x, int T, int d, uint8_t* xq, uint8_t* xs,
                          hipStream_t st) {
  const int nb = d / 32;
  const int nq = T * d / 8;  // eighth-blocks (d % 32 == 0: a block never spans threads of two waves)
  if (nq <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_x_kernel, dim3((nq + 255) / 256), dim3(256), 0, st, x, nq, xq,
                     xq + (size_t)T * d, xs, xs + (size_t)T * nb);
  return hipGetLastError();
}

// ------------------------------------------------------------- MFMA helpers
__device__ __forceinline__ v8i fp4_operand(const v4i q) {
  v8i a = {q[0], q[1], q[2], q[3], 0, 0, 0, 0};
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

// ------------------------------------------------------------- pair slots
// The down GEMM's per-pair outputs wait in HBM for the combine as 24-bit
// floats: the top 24 bits of the fp32 value (sign, 8-bit exponent, 15
// mantissa bits), rounded to nearest (ties away from zero); a NaN stays a
// quiet NaN, and a value that rounds past the largest becomes infinite.
// Relative error <= 2^-16, three quarters of the fp32 bytes.
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t f32_to_f24(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 8) | 0x4000u;  // NaN, kept quiet
  return (u + 0x80u) >> 8;
}
__device__ __forceinline__ float f24_to_f32(uint32_t b) { return __uint_as_float(b << 8); }

// four values -> 12 bytes (three dwords, value 0 in the low bytes)
__device__ __forceinline__ void pack4_f24(const v4f v, uint32_t* w) {
  const uint32_t a = f32_to_f24(v[0]), b = f32_to_f24(v[1]), c = f32_to_f24(v[2]),
                 d = f32_to_f24(v[3]);
  w[0] = a | (b << 24);
  w[1] = (b >> 8) | (c << 16);
  w[2] = (c >> 16) | (d << 8);
}
__device__ __forceinline__ void unpack4_f24(const uint32_t* w, float* v) {
  v[0] = f24_to_f32(w[0] & 0xffffffu);
  v[1] = f24_to_f32((w[0] >> 24) | ((w[1] & 0xffffu) << 8));
  v[2] = f24_to_f32((w[1] >> 16) | ((w[2] & 0xffu) << 16));
  v[3] = f24_to_f32(w[2] >> 8);
}

// ------------------------------------------------------------- grouped GEMM
// One workgroup = 4 waves = one (tile, row block): up to kTileM = 96 tokens
// of one expert (a tile of the grouped pairs) times a block of weight rows.
// At the long-prefill shapes an expert holds 50-100 tokens, so a tile is
// nearly always a whole expert and its weights are read from HBM once
// (96-token tiles leave room for a deeper weight ring than 128-token ones).
//   gate/up (kGateUp): 128 features = 128 gate rows + the same 128 up rows;
//   down    (kDown):   256 output rows.
// Wave w owns 32 features (gate/up: two 16-row MFMA tiles of gate and the
// same two of up, so SwiGLU pairs sit in one lane) or 64 rows (down: four
// 16-row tiles), for all 96 tokens of the tile (six 16-column MFMA tiles).
// No two loads of a workgroup read the same bytes: a request for a line
// that is still in flight stalls the CU's load path.
//
// Two workgroups share a CU (51 KB of LDS and at most 256 registers per
// lane each), so one computes while the other waits for memory. K is walked
// one 128-column tile at a time:
//  - weights (tiled layout, layout.hip) go straight to registers through a
//    ring of kWStages register sets, issued three tiles ahead: one MFMA A
//    operand is one 1 KB tile, one coalesced 16-byte-per-lane buffer load; a
//    scale dword per lane covers 4 K tiles and is fetched with the group's
//    first;
//  - activations (two E4M3 terms + scales) of the tile's tokens are copied
//    once per workgroup straight into LDS (buffer loads to LDS, two stages,
//    one tile ahead; 16-byte piece p of token row t at slot p ^ (t % 8), so
//    the 16 lanes of an MFMA column group read distinct bank groups).
// Every wave issues the same number of loads per step, so a stage is known
// complete by waiting on the wave's load counter down to the count issued
// after it (s_waitcnt vmcnt(N)), followed by a plain workgroup barrier; the
// loads of the next stages stay in flight across it (a __syncthreads would
// wait for all of them).
constexpr int kGateUp = 0;
constexpr int kDown = 1;
constexpr int kStages = 2;                 // activation ring depth (LDS buffers)
constexpr int kWStages = 4;                // weight ring depth (register sets)
constexpr int kActRow = 128;               // LDS bytes per token row and term (one K tile)
constexpr int kScRow = 4;                  // scale bytes per token row and term (4 blocks)
constexpr int kThreads = 256;

template <int MODE>
struct GemmShape {
  static constexpr int NM = (MODE == kGateUp) ? 2 : 1;   // weight matrices
  static constexpr int NRT = (MODE == kGateUp) ? 2 : 4;  // 16-row tiles per matrix per wave
  static constexpr int kRowsPerWave = NRT * 16;           // output rows (features) per wave
  static constexpr int kRowsPerBlock = 4 * kRowsPerWave;  // output rows per workgroup
};

// Loads (vector-memory instructions) one wave issues in the step that
// computes tile c, in order: kActOps activation copies of tile c + 1
// (kActGroups row groups + 1 scale copy), then kWOps weight tiles of tile
// c + kWStages - 1, then, when that tile starts a group of 4, kWOps scale
// dwords for the group. The order is pinned (compiler barriers around each
// group); where in the step they go depends on the tile's size (K loop).
constexpr int kActGroups = kTileM * 2 / 8 / 4;  // 8-row groups per wave (2 terms, 4 waves)
constexpr int kScRows = 128;  // scale rows per term in LDS: two waves copy 64 each (rows past
                              // the tile's tokens read nothing)
constexpr int kActOps = kActGroups + 1;
// column tiles (of 16 tokens) from which a workgroup interleaves its loads
// with its MFMAs (the K loop below)
constexpr int kSpreadMinCols = 4;
constexpr int kWOps = 4;  // NM * NRT for both modes
// Counted at the top of the step that computes tile c (P = c % 8): tile c's
// copies went out one step earlier, followed only by the weights of tile
// c + kWStages - 2 (and their group's scale dwords when that tile starts a
// group). Copies complete in issue order with the other loads, so waiting
// for the counter to drop to this value means the wave's copies of tile c
// have landed in LDS; tile c's own weights, issued before them, have too.
template <int P>
constexpr int loads_after_act() {
  return kWOps + (((P + kWStages - 2) & 3) == 0 ? kWOps : 0);
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt 7 and lgkmcnt 15 mean "do not wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Keeps the machine scheduler from moving instructions across this point.
__device__ __forceinline__ void issue_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Returns its (wave-uniform) argument through a volatile asm statement. A
// load whose address uses the result cannot be issued before the copies that
// precede the call: the asm stays ordered after them, and the load depends on
// it. (Loads may still be issued later than counted, which only makes the
// counted waits stricter.)
__device__ __forceinline__ int after_copies(int v) {
  v = __builtin_amdgcn_readfirstlane(v);
  asm volatile("" : "+s"(v));
  return v;
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding load); the caller has already waited for the
// loads the other waves need.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

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
  uint8_t a[2][kTileM][kActRow];  // activation terms of one K tile, swizzled
  uint8_t s[2][kScRows][kScRow];  // their E8M0 scales, one per 32-column block
};

template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void mx_gemm_kernel(
    int K, int nrows, int f_out, int k, const uint8_t* __restrict__ wq0,
    const uint8_t* __restrict__ ws0, const uint8_t* __restrict__ wq1,
    const uint8_t* __restrict__ ws1, const uint8_t* __restrict__ act_hi,
    const uint8_t* __restrict__ act_lo, const uint8_t* __restrict__ acts_hi,
    const uint8_t* __restrict__ acts_lo, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, int nrb, uint32_t act_bytes, uint8_t* __restrict__ out_hi,
    uint8_t* __restrict__ out_lo, uint8_t* __restrict__ outs_hi, uint8_t* __restrict__ outs_lo,
    uint8_t* __restrict__ slots) {
  using G = GemmShape<MODE>;
  constexpr int NM = G::NM, NRT = G::NRT;
  constexpr int NCT = kTileM / 16;  // 16-token MFMA column tiles per wave
  // separately named buffers (not an array indexed by a runtime number) so
  // reads of one need not wait for the direct-to-LDS copies filling others
  __shared__ __attribute__((aligned(16))) ActLds lds0;
  __shared__ __attribute__((aligned(16))) ActLds lds1;
  __shared__ int tok_lds[kTileM];

  int tile, rb;
  block_coords(nrb, ntiles[0], tile, rb);
  TileInfo ti;
  if (!load_tile(tile, tiles, ntiles, offsets, ti)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int r = lane & 15, g = lane >> 4;
  const int nb = K >> 5, KT = K >> 7, KG = (KT + 3) >> 2, RT = nrows >> 4;
  const int row_base = rb * G::kRowsPerBlock;        // first output row of the block
  const int w0 = row_base + wave * G::kRowsPerWave;   // first output row of this wave
  constexpr int m0 = 0;                               // first tile token of this wave
  const int nct = min(NCT, (ti.cnt + 15) >> 4);       // token tiles holding tokens
  const bool wave_on = w0 < nrows;

  // activation row (token for gate/up, sorted pair position for down) per
  // tile row; rows past the tile's tokens repeat row 0 (loaded, never stored)
  if (tid < kTileM) {
    const int i = (tid < ti.cnt) ? tid : 0;
    tok_lds[tid] = (MODE == kGateUp) ? perm[ti.base + ti.row0 + i] / k : ti.base + ti.row0 + i;
  }
  __syncthreads();

  // ---- weights: tile (rt, kt) of matrix m at wq[m] + ((e RT + rt) KT + kt) 1024 + 16 lane.
  // A wave past the last row loads (and ignores) the first rows instead, so
  // every wave issues the same loads.
  // Weight loads go through a buffer over the wave's NRT row tiles, so the
  // ring's look-ahead past the last K tile reads nothing (an offset past the
  // buffer returns zeros without a memory access). Weights are read once:
  // they are loaded non-temporal so they do not evict the activations, which
  // every row block of the tile reads again, from the L2.
  const int rt0 = (wave_on ? w0 : 0) >> 4;
  constexpr uint32_t kNoRead = 0x7fff0000u;  // beyond any buffer here (all < 2^31 - 2^16)
  __amdgpu_buffer_rsrc_t wq_rs[NM];
  const uint32_t* ws_t[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const uint8_t* q = (m == 0) ? wq0 : wq1;
    const uint8_t* sc = (m == 0) ? ws0 : ws1;
    wq_rs[m] = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(q + (((size_t)ti.e * RT + rt0) * KT) * 1024), 0, NRT * KT * 1024,
        0x00020000);
    ws_t[m] = reinterpret_cast<const uint32_t*>(sc + (((size_t)ti.e * RT + rt0) * KG) * 256) + lane;
  }
  struct WStage {
    v4i q[NM][NRT];
  };
  auto w_issue = [&](int kt, WStage& ws) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
        ws.q[m][rt] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(
                     wq_rs[m], kt < KT ? 16 * lane + (rt * KT + kt) * 1024 : (int)kNoRead, 0, kNonTemporal));
  };
  // scale dwords of groups of 4 K tiles: even groups in sa, odd groups in sb
  // (two named sets, each live across the loop, so no copy is needed)
  int sa[NM][NRT], sb[NM][NRT];
  auto s_issue = [&](int kg, int (&dst)[NM][NRT]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) dst[m][rt] = (int)ws_t[m][((size_t)rt * KG + kg) * 64];
  };

  // ---- activations: wave w copies term w / 2, token rows 64 (w % 2) .. +63
  // as 8 row groups of 8 (lane -> row + lane / 8, slot lane % 8 holding piece
  // slot ^ (row % 8)). A row group past the tile's tokens is given an offset
  // beyond the buffer: the copy then reads nothing and writes zeros, so no
  // copy sits behind a branch and none repeats another's bytes. Scales: wave
  // w copies rows 64 (w / 2) .. +63 of term w % 2 (4 bytes per lane).
  const int term = wave >> 1;
  const int rbase = (kTileM / 2) * (wave & 1);
  // buffer resources over the activation planes (MUBUF copies, bounds-checked
  // against the plane size; word 3 = 32-bit data format, as untyped buffer
  // loads on this family require)
  const __amdgpu_buffer_rsrc_t act_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(term ? act_lo : act_hi), 0, (int)act_bytes, 0x00020000);
  const int sterm = wave & 1;
  const int srow0 = 64 * (wave >> 1);
  const __amdgpu_buffer_rsrc_t sc_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(sterm ? acts_lo : acts_hi), 0, (int)(act_bytes >> 5), 0x00020000);
  uint32_t asrc[kActGroups];
#pragma unroll
  for (int i = 0; i < kActGroups; ++i) {
    const int row = rbase + 8 * i + (lane >> 3);
    asrc[i] = (rbase + 8 * i < ti.cnt)
                  ? (uint32_t)tok_lds[row] * (uint32_t)K + 16u * (uint32_t)((lane & 7) ^ (row & 7))
                  : kNoRead;
  }
  const int srow = srow0 + lane;
  const uint32_t sc_off = srow < ti.cnt ? (uint32_t)tok_lds[srow] * (uint32_t)nb : kNoRead;
  auto act_issue = [&](ActLds& L, int kt) __attribute__((always_inline)) {
    const int kb = kt * 128;
#pragma unroll
    for (int i = 0; i < kActGroups; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(act_rs, (lds_ptr)&L.a[term][rbase + 8 * i][0], 16,
                                               (int)asrc[i], kb, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sc_rs, (lds_ptr)&L.s[sterm][srow0][0], 4, (int)sc_off,
                                             4 * kt, 0, 0);
  };
  // the same copies one row group at a time (i = kActGroups: the scales)
  auto act_issue_one = [&](ActLds& L, int kt, int i) __attribute__((always_inline)) {
    if (i < kActGroups)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(act_rs, (lds_ptr)&L.a[term][rbase + 8 * i][0], 16,
                                               (int)asrc[i], kt * 128, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sc_rs, (lds_ptr)&L.s[sterm][srow0][0], 4,
                                               (int)sc_off, 4 * kt, 0, 0);
  };
  // one step's loads: the copy of tile ka (clamped to the last tile so the
  // tail issues the same loads; that stage is never read), then the weights
  // of tile kw (nothing past the last tile)
  auto stage_issue = [&](ActLds& L, int ka, WStage& ws, int kw) __attribute__((always_inline)) {
    ka = min(ka, KT - 1);
    issue_fence();
    act_issue(L, ka);
    issue_fence();
    w_issue(after_copies(kw), ws);
    issue_fence();
  };

  auto k_loop = [&](auto sp) __attribute__((always_inline)) {
    v4f acc[NM][NRT][NCT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[m][rt][ct] = (v4f){0.f, 0.f, 0.f, 0.f};

    // B operands of one 16-token column tile: pieces g and 4 + g of the token
    // row (K slots 16g.. and 64 + 16g.. of the MFMA), both terms, and the
    // terms' scales of 32-column block g
    struct BFrag {
      v8i hi, lo;
      int shi, slo;
    };
    auto b_load = [&](const ActLds& L, int ct, BFrag& b) __attribute__((always_inline)) {
      const int tr = m0 + 16 * ct + r;
      const int c0 = 16 * (g ^ (r & 7)), c1 = 16 * ((4 + g) ^ (r & 7));
      b.hi = fp8_operand(*reinterpret_cast<const uint4*>(&L.a[0][tr][c0]),
                         *reinterpret_cast<const uint4*>(&L.a[0][tr][c1]));
      b.lo = fp8_operand(*reinterpret_cast<const uint4*>(&L.a[1][tr][c0]),
                         *reinterpret_cast<const uint4*>(&L.a[1][tr][c1]));
      b.shi = L.s[0][tr][g];
      b.slo = L.s[1][tr][g];
    };
    // one K tile of MFMAs; P = the tile's byte in the weight scale dwords. The
    // next column tile's B operands are read while this one's MFMAs run.
    auto compute = [&](const ActLds& L, const WStage& ws, const int (&sw)[NM][NRT], auto pc,
                       auto&& piece) __attribute__((always_inline)) {
      constexpr int P = decltype(pc)::value;
      BFrag b[2];
      b_load(L, 0, b[0]);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        piece(ct);  // loads issued ahead of this column tile (if any)
        // The next column tile's B reads go out whether or not it holds
        // tokens (its rows are inside the stage; the values of an empty one
        // go unused). Behind a branch on that tile's tokens, the compiler could
        // not tell how many LDS reads follow this tile's and waited for all
        // of them before this tile's MFMAs (measured: gate/up 0.6%, down
        // 0.8% faster).
        if (ct + 1 < NCT) b_load(L, ct + 1, b[(ct + 1) & 1]);
        if (ct < nct) {
          const BFrag& cb = b[ct & 1];
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
              acc[m][rt][ct] =
                  mfma_fp4_fp8<P>(fp4_operand(ws.q[m][rt]), sw[m][rt], cb.hi, cb.shi,
                                  acc[m][rt][ct]);
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
              acc[m][rt][ct] =
                  mfma_fp4_fp8<P>(fp4_operand(ws.q[m][rt]), sw[m][rt], cb.lo, cb.slo,
                                  acc[m][rt][ct]);
        }
      }
    };

    // ---- K loop: tile c's activations in LDS buffer c % 2, its weights in
    // register set c % 4 (issued three steps ahead); scale dwords of even
    // groups of 4 tiles in sa, odd groups in sb. Step P (= c % 8): wait for
    // tile c's copies (its weights, issued earlier, have landed too), barrier,
    // issue the copy of tile c + 1 and the weights of tile c + 3 (with that
    // group's scale dwords when c + 3 starts one), compute tile c.
    //
    // Where the step's loads go (SPREAD, fixed per workgroup, so each loop is
    // free of branches on it):
    //  - SPREAD (tiles of at least kSpreadMinCols column tiles): between the
    //    MFMAs, in the order the load counter arithmetic assumes: the copies
    //    of tile c + 1 (clamped as in stage_issue) three, two and two ahead
    //    of column tiles 0, 1 and 2, then the weights of tile c + kWStages - 1
    //    (and that group's scale dwords) ahead of column tile 4 (gate/up;
    //    after the last MFMA of a tile of 4 column tiles) or 3 (down). The
    //    CU's load path then takes a few requests at a time while the matrix
    //    cores stay busy, instead of a burst of 11 or 15 at the top of the
    //    step;
    //  - otherwise all at the top of the step: a tile of few tokens is paced
    //    by its weight stream, and the few MFMAs a later issue would wait for
    //    only delay it.
    // Measured (T = 4096 with skewed routing, and uniform routing at T = 5 to
    // 4096): the layer 2.3% faster at T = 4096 than with every tile issuing at
    // the top, and no slower at any smaller T; interleaving tiles of 1-3 column
    // tiles as well cost 1-3% at T = 5-1024; interleaving only full tiles gained
    // nothing. A branch on the tile size at each issue point (not one per
    // workgroup) cost more than either order gained.
    static_assert(kActOps == 7 && NCT >= 5, "the 3/2/2 split below covers 7 copies");
    auto step = [&](auto pc, auto spread, const ActLds& Lc, const WStage& Wc,
                    const int (&sc)[NM][NRT], ActLds& Ln, WStage& Wn, int c)
        __attribute__((always_inline)) {
      constexpr int P = decltype(pc)::value;
      wait_vmcnt<loads_after_act<P>()>();
      stage_barrier();
      const int kw = c + kWStages - 1;
      auto s_issue_group = [&]() __attribute__((always_inline)) {
        if constexpr (((P + kWStages - 1) & 3) == 0) {
          s_issue(after_copies(min(kw >> 2, KG - 1)), (((P + kWStages - 1) >> 2) & 1) ? sb : sa);
          issue_fence();
        }
      };
      if constexpr (decltype(spread)::value) {
        // the weights' column tile: 4 for gate/up, 3 for down (measured: down
        // 0.5-0.9% faster with 3 than with 4, gate/up slower with 3)
        constexpr int kWeightsAt = MODE == kDown ? 3 : 4;
        const int ka = min(c + 1, KT - 1);
        compute(Lc, Wc, sc, std::integral_constant<int, P & 3>(), [&](int ct) {
          if (ct < 3) {
            issue_fence();
            const int i0 = ct == 0 ? 0 : (ct == 1 ? 3 : 5);
            const int n = ct == 0 ? 3 : 2;
#pragma unroll
            for (int i = 0; i < n; ++i) act_issue_one(Ln, ka, i0 + i);
            issue_fence();
          } else if (ct == kWeightsAt) {
            issue_fence();
            w_issue(after_copies(kw), Wn);
            issue_fence();
            s_issue_group();
          }
        });
      } else {
        stage_issue(Ln, c + 1, Wn, kw);
        s_issue_group();
        compute(Lc, Wc, sc, std::integral_constant<int, P & 3>(), [](int) {});
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;
    using I6 = std::integral_constant<int, 6>;
    using I7 = std::integral_constant<int, 7>;
    static_assert(kWStages == 4 && kStages == 2, "the unrolled ring below assumes these depths");
    WStage wa, wb, wc, wd;
    stage_issue(lds0, 0, wa, 0);
    s_issue(0, sa);
    issue_fence();
    w_issue(1, wb);
    issue_fence();
    w_issue(2, wc);
    issue_fence();
    for (int c = 0; c < KT; c += 8) {
      step(I0(), sp, lds0, wa, sa, lds1, wd, c);
      if (c + 1 >= KT) break;
      step(I1(), sp, lds1, wb, sa, lds0, wa, c + 1);
      if (c + 2 >= KT) break;
      step(I2(), sp, lds0, wc, sa, lds1, wb, c + 2);
      if (c + 3 >= KT) break;
      step(I3(), sp, lds1, wd, sa, lds0, wc, c + 3);
      if (c + 4 >= KT) break;
      step(I4(), sp, lds0, wa, sb, lds1, wd, c + 4);
      if (c + 5 >= KT) break;
      step(I5(), sp, lds1, wb, sb, lds0, wa, c + 5);
      if (c + 6 >= KT) break;
      step(I6(), sp, lds0, wc, sb, lds1, wb, c + 6);
      if (c + 7 >= KT) break;
      step(I7(), sp, lds1, wd, sb, lds0, wc, c + 7);
    }
    // no copy may still be writing this workgroup's LDS when it exits. (A
    // wave past the last row computed on the first rows' weights: discarded.)
    wait_vmcnt<0>();
    if (!wave_on) return;

    if constexpr (MODE == kGateUp) {
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
      // this pair's expert output into the pair's own slot (no atomics; summed
      // per token later; streamed past the caches, it is read once by the
      // combine), as 24-bit floats: the wave's 64 rows of a pair are 192
      // contiguous bytes, 64-byte aligned. Lane (r, g) holds rows
      // 16 rt + 4 g + i of token column r; it packs each block of four rows
      // into 12 bytes of a private LDS slice (one 192-byte row per column),
      // then reads back and stores 16-byte pieces so that each store writes 64
      // contiguous bytes of every column.
      // LDS banks: a column's row starts at dword 52 r + 2 (r / 8), so the 32
      // lanes (r, g < 2) of a half-wave's dword writes (dword 52 r + 3 g + ...
      // modulo 32 banks) hit 32 distinct banks; without the 2-dword shift
      // columns r and r + 8 would share banks. The shift leaves rows 8-byte
      // aligned, so they are read back in 8-byte halves.
      static_assert(NRT == 4, "the slot layout assumes four row tiles per wave");
      constexpr int kStRow = 192 + 16;  // bytes per column (room for the shift)
      __shared__ __attribute__((aligned(16))) uint32_t st_all[4][16 * kStRow / 4];
      uint8_t* st = reinterpret_cast<uint8_t*>(st_all[wave]);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        if (ct >= nct) continue;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          uint32_t w[3];
          pack4_f24(acc[0][rt][ct], w);
          uint32_t* dst =
              reinterpret_cast<uint32_t*>(st + r * kStRow + 8 * (r >> 3) + 48 * rt + 12 * g);
          dst[0] = w[0];
          dst[1] = w[1];
          dst[2] = w[2];
        }
        v4u32 piece[3];  // bytes 64 q + 16 g .. + 15 of column r's 192
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          const uint8_t* src = st + r * kStRow + 8 * (r >> 3) + 64 * q + 16 * g;
          const uint2 a = *reinterpret_cast<const uint2*>(src);
          const uint2 b = *reinterpret_cast<const uint2*>(src + 8);
          piece[q] = (v4u32){a.x, a.y, b.x, b.y};
        }
        const int i = m0 + 16 * ct + r;
        if (i < ti.cnt) {
          const int pair = perm[ti.base + ti.row0 + i];
          uint8_t* o = slots + ((size_t)pair * nrows + w0) * 3 + 16 * g;
#pragma unroll
          for (int q = 0; q < 3; ++q)
            __builtin_nontemporal_store(piece[q], reinterpret_cast<v4u32*>(o + 64 * q));
        }
      }
    }
  };  // k_loop: each schedule has its own accumulators, drain and epilogue
  // (the choice through a scalar register: the compiler does not know nct is
  // uniform, and a masked branch here would run both loops' registers at once)
  if (__builtin_amdgcn_readfirstlane(nct) >= kSpreadMinCols)
    k_loop(std::true_type());
  else
    k_loop(std::false_type());
}

// y[t] = sum_j gate[t,j] * slot[t*k + j], j in order; pairs whose expert is
// outside [0, E) contribute zero. One thread per 4 outputs (12 contiguous
// bytes of a slot, so a wave's loads are contiguous).
typedef uint32_t v3u32 __attribute__((ext_vector_type(3), aligned(4)));

__global__ __launch_bounds__(256) void combine_kernel(const uint8_t* __restrict__ slots,
                                                      const int32_t* __restrict__ idx,
                                                      const float* __restrict__ gate, int T,
                                                      int d, int k, int E, float* __restrict__ y) {
  const int d4 = d >> 2;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)T * d4) return;
  const int t = (int)(i / d4), c = (int)(i % d4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // every slot and gate is read (a dropped pair's slot is allocated but
  // unwritten and its values are replaced by zero, not multiplied), so the
  // loop has no branch and the loads of all its slots are in flight together
  // (a gate read only for a kept pair made one branch per slot, and the
  // compiler waited for the loads at each: 8% slower)
#pragma unroll 16
  for (int j = 0; j < k; ++j) {
    const int e = idx[(size_t)t * k + j];
    const float g = gate[(size_t)t * k + j];
    const bool on = e >= 0 && e < E;
    const float gw = on ? g : 0.0f;
    const v3u32 w3 = __builtin_nontemporal_load(
        reinterpret_cast<const v3u32*>(slots + (((size_t)t * k + j) * d + 4 * (size_t)c) * 3));
    const uint32_t w[3] = {w3[0], w3[1], w3[2]};
    float v[4];
    unpack4_f24(w, v);
    if (!on) v[0] = v[1] = v[2] = v[3] = 0.0f;
    acc.x = fmaf(gw, v[0], acc.x);
    acc.y = fmaf(gw, v[1], acc.y);
    acc.z = fmaf(gw, v[2], acc.z);
    acc.w = fmaf(gw, v[3], acc.w);
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
                     xs, xs + xsplane, offsets, perm, tiles, ntiles, nrb, (uint32_t)xplane, hq, hq + hplane, hs,
                     hs + hsplane, nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm_down(int T, const Shape& s, const ExpertWeights& w, const int32_t* offsets,
                            const int32_t* perm, const int32_t* tiles, const int32_t* ntiles,
                            int max_tiles, const uint8_t* hq, const uint8_t* hs, uint8_t* slots,
                            hipStream_t st) {
  if (T <= 0 || max_tiles <= 0) return hipSuccess;
  const size_t P = (size_t)T * s.k;
  const size_t hplane = P * s.f, hsplane = P * (s.f / 32);
  constexpr int rpb = GemmShape<kDown>::kRowsPerBlock;
  const int nrb = (s.d + rpb - 1) / rpb;
  hipLaunchKernelGGL(mx_gemm_kernel<kDown>, dim3(gemm_grid(max_tiles, nrb)), dim3(kThreads), 0,
                     st, s.f, s.d, s.f, s.k, w.down_q, w.down_s, nullptr, nullptr, hq, hq + hplane,
                     hs, hs + hsplane, offsets, perm, tiles, ntiles, nrb, (uint32_t)hplane, nullptr, nullptr, nullptr,
                     nullptr, slots);
  return hipGetLastError();
}

hipError_t launch_combine(const uint8_t* slots, const int32_t* idx, const float* gate, int T,
                          const Shape& s, float* y, hipStream_t st) {
  const size_t n = (size_t)T * (s.d / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, slots,
                     idx, gate, T, s.d, s.k, s.E, y);
  return hipGetLastError();
}

}  // namespace k3
