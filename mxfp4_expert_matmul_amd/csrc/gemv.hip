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
#include <type_traits>
#include <utility>

#include "k3_device.h"
#include "k3_kernels.h"
#include "topk_device.h"

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

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
// Expert weights are read once per call: their buffer loads are streamed
// (non-temporal), so they do not push the router weights and activations out
// of the caches.
constexpr int kNonTemporal = 2;

// Both GEMVs stream weights through rings of register sets filled by buffer
// loads whose count per step is fixed, and wait on the load counter with
// s_waitcnt vmcnt(N) (N = loads issued after the ones needed); the fences
// keep the compiler from moving loads across those points.
template <int N>
__device__ __forceinline__ void gemv_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt on the LDS counter only (lgkmcnt(0); vmcnt and expcnt at their
// "do not wait" values)
__device__ __forceinline__ void gemv_wait_lds() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
}
__device__ __forceinline__ void gemv_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
template <int V>
using ic = std::integral_constant<int, V>;
// f(ic<0>{}), f(ic<1>{}), ..., f(ic<N - 1>{}): compile-time indices
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F& f, std::integer_sequence<int, I...>) {
  (f(ic<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// gate/up: one wave per (pair, 16-row tile of gate and of up); the four
// waves of a workgroup serve one pair. With `logits` given (the whole-layer
// call) wave 0 first loads its token's logits, every wave then copies its
// share of the token's x (bf16) into the workgroup's LDS (buffer loads to
// LDS, one copy per workgroup), and wave 0 selects the token's top k (the
// same selection as the top-k kernel, waiting for the logits alone) and
// passes its pair's expert to the other waves through LDS, so no top-k
// launch sits between the router and this kernel; the workgroup of slot 0
// and row block 0 writes the token's idx and gates for the down GEMV and the
// caller. Otherwise idx is the caller's routing. The wave then walks K four 128-column tiles per step with the
// next kGuDepth - 1 steps' weights in flight (ten buffer loads per step:
// four 1 KB tiles of gate, four of up, one scale dword of each; past the
// last tile they read zeros without touching memory); one barrier before
// the first step's compute makes the whole x visible. Lane (r, g) takes row
// 16 rt + r, K block g of every tile, so one 16-byte load per lane reads a
// whole 1 KB tile; its 32 activations are the same for the 16 lanes of a
// group (an LDS broadcast). Rows are summed over the 4 groups at the end.
// grid: (T*k pairs, ceil(f / 64)), block 256 (4 waves = 4 row tiles),
// dynamic LDS (XC + 1) KB.
constexpr int kGuTiles = 4;
constexpr int kGuDepth = 3;
constexpr int kGuLoads = 2 * kGuTiles + 2;

// 1 KB pieces of x (d <= 512 XC; bytes past d read as zeros)
__host__ __device__ constexpr int gu_x_copies(int d) {
  return d <= 1024 ? 2 : d <= 2048 ? 4 : d <= 4096 ? 8 : d <= 7168 ? 14 : 16;
}

template <int XC, int V>  // V: logits per lane in the selection, E <= 64 V
__global__ __launch_bounds__(256) void gemv_gateup_kernel(
    const uint16_t* __restrict__ x, int d, int f, int k, int E, const uint8_t* __restrict__ gq,
    const uint8_t* __restrict__ gs, const uint8_t* __restrict__ uq, const uint8_t* __restrict__ us,
    const float* __restrict__ logits, const float* __restrict__ sel_bias,
    int32_t* __restrict__ idx, float* __restrict__ gate,
    float* __restrict__ h32) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xl[];  // [512 * XC] + a 1 KB dump
  __shared__ __attribute__((aligned(16))) uint64_t cand[kTopkCand];
  __shared__ uint64_t sel[64];
  __shared__ int pair_expert;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int pair = blockIdx.x;
  const int rt = blockIdx.y * 4 + wave;
  const int RT = f >> 4, KT = d >> 7, KG = (KT + 3) >> 2;
  const int t = pair / k, j = pair - t * k;
  // the token's logits first: the selection then waits for them alone, not
  // for the x copies issued after them
  const float* lrow = logits ? logits + (size_t)t * E : nullptr;
  TopkRow<V> rw;
  if (logits && wave == 0) topk_load<V>(lrow, E, sel_bias, rw);
  uint16_t* xw = xl;
  {  // x once per workgroup (all four waves serve one pair): wave w copies
     // 1 KB pieces w, w + 4, ...; a piece number past x's end goes to the
     // dump kilobyte and reads nothing
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x + (size_t)t * d), 0, 2 * d, 0x00020000);
    constexpr int kPer = (XC + 3) / 4;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int v = wave + 4 * i;
      const bool in = v < XC;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_ptr)(xl + 512 * (in ? v : XC)), 16,
                                               in ? 16 * lane + 1024 * v : (int)0x7fff0000, 0, 0, 0);
    }
  }
  int e;
  if (logits) {
    // wave 0 selects for the workgroup (all four waves serve one pair), the
    // others take the pair's expert from LDS after a barrier
    if (wave == 0) {
      const uint64_t mine = topk_select<V>(rw, sel_bias != nullptr, E, k, cand, sel);
      if (lane == 0) pair_expert = ~__builtin_amdgcn_readlane((int)(uint32_t)mine, j);
      if (j == 0 && blockIdx.y == 0) {
        const float g = sel_bias ? topk_gate_unbiased(mine, k, lrow) : topk_gate_of(mine, k);
        if (lane < k) {
          idx[(size_t)t * k + lane] = topk_key_index(mine);
          gate[(size_t)t * k + lane] = g;
        }
      }
      gemv_wait_lds();  // the expert is in LDS (the x copies may still be in flight)
    }
    gemv_fence();
    __builtin_amdgcn_s_barrier();
    gemv_fence();
    e = __builtin_amdgcn_readfirstlane(pair_expert);
  } else {
    e = idx[pair];
    if (e < 0 || e >= E) {  // dropped pair (the whole workgroup): never read downstream
      gemv_wait_vmcnt<0>();  // no copy may still be writing this workgroup's LDS
      return;
    }
  }
  if (rt >= RT) {  // past the last row tile: the copies and the barrier only
    gemv_wait_vmcnt<0>();
    gemv_fence();
    __builtin_amdgcn_s_barrier();
    return;
  }
  // buffers over this row tile's K tiles (codes) and scale groups
  const size_t row = (size_t)e * RT + rt;
  const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(gq + row * KT * 1024), 0, KT * 1024, 0x00020000);
  const __amdgpu_buffer_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(uq + row * KT * 1024), 0, KT * 1024, 0x00020000);
  const __amdgpu_buffer_rsrc_t rgs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(gs + row * KG * 256), 0, KG * 256, 0x00020000);
  const __amdgpu_buffer_rsrc_t rus = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(us + row * KG * 256), 0, KG * 256, 0x00020000);
  struct Ring {
    v4u qg[kGuTiles], qu[kGuTiles];
    uint32_t sg, su;
  };
  // step s: K tiles 4s .. 4s + 3 and their scale group s (offsets past the
  // buffers read zeros). The per-lane offsets pass through an asm statement
  // at the issue point, so no load can be hoisted above it: the compiler does
  // not order these buffer loads against the fences' memory clobbers.
  auto issue = [&](int s, Ring& b) {
    int vq = 16 * lane, vs = 4 * lane;
    asm volatile("" : "+v"(vq), "+v"(vs));
#pragma unroll
    for (int i = 0; i < kGuTiles; ++i) {
      b.qg[i] = __builtin_amdgcn_raw_buffer_load_b128(rg, vq + 1024 * (4 * s + i), 0, kNonTemporal);
      b.qu[i] = __builtin_amdgcn_raw_buffer_load_b128(ru, vq + 1024 * (4 * s + i), 0, kNonTemporal);
    }
    b.sg = __builtin_amdgcn_raw_buffer_load_b32(rgs, vs + 256 * s, 0, 0);
    b.su = __builtin_amdgcn_raw_buffer_load_b32(rus, vs + 256 * s, 0, 0);
  };
  float ga = 0.0f, ua = 0.0f;
  auto compute = [&](int s, const Ring& b) {
#pragma unroll
    for (int i = 0; i < kGuTiles; ++i) {
      const int kt = 4 * s + i;
      if (kt < KT) {
        const uint4* xs = reinterpret_cast<const uint4*>(xw + 128 * kt + 32 * g);
        uint32_t xv[16];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 q = xs[v];
          xv[4 * v] = q.x; xv[4 * v + 1] = q.y; xv[4 * v + 2] = q.z; xv[4 * v + 3] = q.w;
        }
        const uint4 qg = {b.qg[i].x, b.qg[i].y, b.qg[i].z, b.qg[i].w};
        const uint4 qu = {b.qu[i].x, b.qu[i].y, b.qu[i].z, b.qu[i].w};
        ga = fmaf(block_dot_bf16(qg, xv), e8m0_to_f32((b.sg >> (8 * i)) & 0xffu), ga);
        ua = fmaf(block_dot_bf16(qu, xv), e8m0_to_f32((b.su >> (8 * i)) & 0xffu), ua);
      }
    }
  };
  // K fully unrolled (XC >= KG steps), so the ring's register sets are fixed
  // at compile time; steps past the last read zeros and compute nothing
  Ring ring[kGuDepth];
  gemv_fence();
  static_for<kGuDepth - 1>([&](auto P) {
    issue(P(), ring[P()]);
    gemv_fence();  // one step's loads, tiles then scales, before the next step's
    // A second use of the step's registers in a branch that is never taken
    // (KT >= 1): with uses in two blocks the compiler cannot sink the loads
    // into the first compute's bounds branch, after the later steps' loads.
    if (KT < 0) {
      const Ring& b = ring[P()];
      asm volatile("" ::"v"(b.qg[0]), "v"(b.qg[1]), "v"(b.qg[2]), "v"(b.qg[3]), "v"(b.qu[0]),
                   "v"(b.qu[1]), "v"(b.qu[2]), "v"(b.qu[3]), "v"(b.sg), "v"(b.su));
    }
  });
  static_for<XC>([&](auto S) {
    constexpr int s = S();
    gemv_fence();
    if constexpr (s + kGuDepth - 1 < XC) issue(s + kGuDepth - 1, ring[(s + kGuDepth - 1) % kGuDepth]);
    gemv_fence();
    // step s's loads (and x, issued before all of them) have landed
    constexpr int after = (XC - 1 - s < kGuDepth - 1 ? XC - 1 - s : kGuDepth - 1) * kGuLoads;
    gemv_wait_vmcnt<after>();
    gemv_fence();
    if constexpr (s == 0) {  // every wave's pieces of x have landed
      __builtin_amdgcn_s_barrier();
      gemv_fence();
    }
    if (4 * s < KT) compute(s, ring[s % kGuDepth]);
  });
  gemv_wait_vmcnt<0>();
  ga += __shfl_xor(ga, 16, 64);
  ga += __shfl_xor(ga, 32, 64);
  ua += __shfl_xor(ua, 16, 64);
  ua += __shfl_xor(ua, 32, 64);
  if (g == 0) h32[(size_t)pair * f + 16 * rt + r] = silu_f32(ga) * ua;
}

// down + combine: workgroup = one token x two 16-row tiles of the output; its
// 16 waves take one slot each (wave w: j = w, w + 16, ...). A wave copies its
// slot's h (fp32, up to 2048 values: one "piece" of K) straight into its own
// LDS region (buffer loads to LDS) and then walks 4-tile steps over both row
// tiles with the weights of the next kDownDepth - 1 steps in flight (a ring
// of register sets). Every step issues the same five buffer loads (four 1 KB
// tiles and one scale dword per lane); a load past the row tile's K extent
// or of a dropped slot is given an empty buffer and reads zeros without
// touching memory (the whole offset is in the per-lane part, which the
// buffer's size check covers), so the counted waits below are exact. With
// k <= 16 and f <= 2048 the h copy is the wave's first load and no step
// waits for it; otherwise h is copied again at every (slot, piece) segment.
// Each 32-value block of h is read back as an LDS broadcast. Lane (r, g)
// keeps gate-weighted partials of rows 16 rt + r over K block g of every
// tile; partials meet across lane groups, then across waves in fixed order.
// Deterministic, no atomics.
// grid: (T, d / 32), block 1024, dynamic LDS 16 waves x 2 KB x NCP.
constexpr int kDownTiles = 4;  // K tiles per step
constexpr int kDownWaves = 16;
constexpr int kDownDepth = 4;  // ring of weight register sets
constexpr int kDownLoads = kDownTiles + 1;
constexpr int kDownPiece = 2048;  // h values staged at once per wave (8 KB)

// 4-tile chunks per h piece (a piece is min(f, 2048) values, <= 512 NCP)
__host__ __device__ constexpr int down_piece_chunks(int f) {
  return f <= 512 ? 1 : f <= 1024 ? 2 : 4;
}

// MULTI: more than one (slot, piece) segment per wave (k > 16 or f > 2048)
template <int NCP, bool MULTI>
__global__ __launch_bounds__(64 * kDownWaves) void gemv_down_kernel(
    int d, int f, int k, int E, const uint8_t* __restrict__ dq, const uint8_t* __restrict__ ds,
    const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const float* __restrict__ h32, float* __restrict__ y) {
  constexpr int SPS = 2 * NCP;                                 // steps per segment
  constexpr int DEPTH = SPS < kDownDepth ? SPS : kDownDepth;  // ring depth
  static_assert(SPS % DEPTH == 0, "ring phase must repeat every segment");
  constexpr int HP = 512 * NCP;  // h values per piece (= LDS floats per wave)
  extern __shared__ __attribute__((aligned(16))) float hl[];  // [kDownWaves][HP]
  __shared__ float red[kDownWaves][32];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int t = blockIdx.x, rp = blockIdx.y;  // row tiles 2 rp, 2 rp + 1
  const int RT = d >> 4, KT = f >> 7, KG = (KT + 3) >> 2;
  const int npiece = (f + kDownPiece - 1) / kDownPiece;
  float* hw = hl + (size_t)wave * HP;
  struct Ring {
    v4u q[kDownTiles];
    uint32_t sw;
  };
  const int nslot = (k - wave + kDownWaves - 1) / kDownWaves;  // slots wave, wave + 16, ...
  const int nseg = nslot * npiece;
  // expert of the wave's i-th slot, -1 past the last slot or for a dropped pair
  auto expert_of = [&](int i) {
    if (i >= nslot) return -1;
    const int e = idx[(size_t)t * k + wave + kDownWaves * i];
    return (e >= 0 && e < E) ? e : -1;
  };
  // step u of segment sg: row tile 2 rp + u / NCP, K tiles from
  // 16 piece + 4 (u % NCP) (a piece is 16 K tiles)
  auto issue = [&](int sg, int u, Ring& b) {
    const int e = sg < nseg ? expert_of(sg / npiece) : -1;
    const int kt0 = (kDownPiece / 128) * (sg % npiece) + kDownTiles * (u % NCP);
    const bool on = e >= 0;
    const size_t row = on ? (size_t)e * RT + 2 * rp + u / NCP : 0;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(dq + row * KT * 1024), 0, on ? KT * 1024 : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(ds + row * KG * 256), 0, on ? KG * 256 : 0, 0x00020000);
#pragma unroll
    for (int i = 0; i < kDownTiles; ++i)
      b.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, 16 * lane + 1024 * (kt0 + i), 0, kNonTemporal);
    b.sw = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * lane + 256 * (kt0 >> 2), 0, 0);
  };
  // h piece of segment sg -> the wave's LDS region (2 NCP copies of 1 KB;
  // values past f, and segments with nothing to compute, read as zeros)
  auto h_copy = [&](int sg) {
    const bool on = sg < nseg && expert_of(sg / npiece) >= 0;
    const size_t pair = on ? (size_t)t * k + wave + kDownWaves * (sg / npiece) : 0;
    const int p0 = kDownPiece * (sg % npiece);
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(h32 + pair * f + (on ? p0 : 0)), 0, on ? 4 * (f - p0) : 0, 0x00020000);
#pragma unroll
    for (int v = 0; v < 2 * NCP; ++v)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lds_void_ptr)(hw + 256 * v), 16,
                                               16 * lane + 1024 * v, 0, 0, 0);
  };
  float acc0 = 0.0f, acc1 = 0.0f;  // rows of row tile 2 rp and 2 rp + 1
  auto compute = [&](int sg, int u, const Ring& b) {
    const int c = u % NCP;
    const int kt0 = (kDownPiece / 128) * (sg % npiece) + kDownTiles * c;
    float pe = 0.0f;
#pragma unroll
    for (int i = 0; i < kDownTiles; ++i)
      if (kt0 + i < KT) {
        const float4* hs = reinterpret_cast<const float4*>(hw + 128 * (kDownTiles * c + i) + 32 * g);
        float hv[32];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float4 h4 = hs[v];
          hv[4 * v] = h4.x; hv[4 * v + 1] = h4.y; hv[4 * v + 2] = h4.z; hv[4 * v + 3] = h4.w;
        }
        const uint4 q = {b.q[i].x, b.q[i].y, b.q[i].z, b.q[i].w};
        pe = fmaf(block_dot_f32(q, hv), e8m0_to_f32((b.sw >> (8 * i)) & 0xffu), pe);
      }
    const float gw = gate[(size_t)t * k + wave + kDownWaves * (sg / npiece)];
    if (u < NCP)
      acc0 = fmaf(gw, pe, acc0);
    else
      acc1 = fmaf(gw, pe, acc1);
  };
  Ring ring[DEPTH];
  // one segment's steps; its first DEPTH - 1 steps' weights are in flight on
  // entry, and on exit the next segment's first DEPTH - 1 are
  auto segment = [&](int sg) {
    static_for<SPS>([&](auto U) {
      constexpr int u = U();
      constexpr int un = u + DEPTH - 1;  // step issued now: un of sg, or un - SPS of sg + 1
      gemv_fence();
      if constexpr (un < SPS)
        issue(sg, un, ring[un % DEPTH]);
      else
        issue(sg + 1, un - SPS, ring[un % DEPTH]);
      gemv_fence();
      gemv_wait_vmcnt<kDownLoads * (DEPTH - 1)>();  // step u's loads (and before) landed
      gemv_fence();
      if (expert_of(sg / npiece) >= 0) compute(sg, u, ring[u % DEPTH]);
    });
  };
  // the first segment's h, then its first steps' weights
  h_copy(0);
  gemv_fence();
  static_for<DEPTH - 1>([&](auto P) { issue(0, P(), ring[P()]); });
  segment(0);
  if constexpr (MULTI) {
    for (int sg = 1; sg < nseg; ++sg) {
      gemv_fence();
      h_copy(sg);  // every LDS read of the previous segment has completed
      gemv_fence();
      gemv_wait_vmcnt<0>();
      gemv_fence();
      segment(sg);
    }
  }
  gemv_wait_vmcnt<0>();
  acc0 += __shfl_xor(acc0, 16, 64);
  acc0 += __shfl_xor(acc0, 32, 64);
  acc1 += __shfl_xor(acc1, 16, 64);
  acc1 += __shfl_xor(acc1, 32, 64);
  if (g == 0) {
    red[wave][r] = acc0;
    red[wave][16 + r] = acc1;
  }
  __syncthreads();
  if (tid < 32) {
    float s = red[0][tid];
#pragma unroll
    for (int w = 1; w < kDownWaves; ++w) s += red[w][tid];
    y[(size_t)t * d + 32 * rp + tid] = s;
  }
}

static size_t gateup_lds_bytes(int d) { return (size_t)1024 * (gu_x_copies(d) + 1); }

hipError_t launch_gemv_gateup(const uint16_t* x, int T, const Shape& s, const ExpertWeights& w,
                              const float* logits, const float* sel_bias, int32_t* idx,
                              float* gate, float* h32, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const dim3 g1(T * s.k, (s.f / 16 + 3) / 4);
  const size_t lds = gateup_lds_bytes(s.d);
#define K3_GATEUP(XC, V)                                                                       \
  hipLaunchKernelGGL((gemv_gateup_kernel<XC, V>), g1, dim3(256), lds, st, x, s.d, s.f, s.k,   \
                     s.E, w.gate_q, w.gate_s, w.up_q, w.up_s, logits, sel_bias, idx, gate, h32)
#define K3_GATEUP_V(XC)                                                                        \
  do {                                                                                         \
    if (s.E <= 1024)                                                                           \
      K3_GATEUP(XC, 16);                                                                       \
    else                                                                                       \
      K3_GATEUP(XC, 64);                                                                       \
  } while (0)
  switch (gu_x_copies(s.d)) {
    case 2: K3_GATEUP_V(2); break;
    case 4: K3_GATEUP_V(4); break;
    case 8: K3_GATEUP_V(8); break;
    case 14: K3_GATEUP_V(14); break;
    default: K3_GATEUP_V(16); break;
  }
#undef K3_GATEUP_V
#undef K3_GATEUP
  return hipGetLastError();
}

static size_t down_lds_bytes(int ncp) { return (size_t)kDownWaves * 2048 * ncp; }

template <int NCP, bool MULTI>
static hipError_t set_down_lds() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_down_kernel<NCP, MULTI>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)down_lds_bytes(NCP));
}

template <int NCP>
static hipError_t set_down_lds_nc() {
  hipError_t e = set_down_lds<NCP, false>();
  return e != hipSuccess ? e : set_down_lds<NCP, true>();
}

hipError_t prepare_gemv(const Shape& s) {
  const bool v64 = s.E > 1024;
  const void* gu;
  switch (gu_x_copies(s.d)) {
#define K3_GU(XC)                                                                              \
  gu = v64 ? reinterpret_cast<const void*>(gemv_gateup_kernel<XC, 64>)                         \
           : reinterpret_cast<const void*>(gemv_gateup_kernel<XC, 16>)
    case 2: K3_GU(2); break;
    case 4: K3_GU(4); break;
    case 8: K3_GU(8); break;
    case 14: K3_GU(14); break;
    default: K3_GU(16); break;
#undef K3_GU
  }
  const hipError_t e = hipFuncSetAttribute(gu, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)gateup_lds_bytes(s.d));
  if (e != hipSuccess) return e;
  switch (down_piece_chunks(s.f)) {
    case 1: return set_down_lds_nc<1>();
    case 2: return set_down_lds_nc<2>();
    default: return set_down_lds_nc<4>();
  }
}

// Every decode kernel instantiation's dynamic LDS limit. Each limit is fixed by
// the instantiation's template arguments, so this does not depend on a shape.
hipError_t prepare_gemv_all() {
  hipError_t e = hipSuccess;
  auto gu = [&](const void* fn, int xc) {
    if (e == hipSuccess)
      e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                              1024 * (xc + 1));
  };
#define K3_GU_ALL(XC)                                                       \
  gu(reinterpret_cast<const void*>(gemv_gateup_kernel<XC, 16>), XC);        \
  gu(reinterpret_cast<const void*>(gemv_gateup_kernel<XC, 64>), XC)
  K3_GU_ALL(2);
  K3_GU_ALL(4);
  K3_GU_ALL(8);
  K3_GU_ALL(14);
  K3_GU_ALL(16);
#undef K3_GU_ALL
  if (e == hipSuccess) e = set_down_lds_nc<1>();
  if (e == hipSuccess) e = set_down_lds_nc<2>();
  if (e == hipSuccess) e = set_down_lds_nc<4>();
  return e;
}

hipError_t launch_gemv_down(int T, const Shape& s, const ExpertWeights& w, const int32_t* idx,
                            const float* gate, const float* h32, float* y, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const dim3 grid(T, s.d / 32), block(64 * kDownWaves);
  const int ncp = down_piece_chunks(s.f);
  const bool multi = s.k > kDownWaves || s.f > kDownPiece;
  const size_t lds = down_lds_bytes(ncp);
#define K3_DOWN(NCP)                                                                           \
  do {                                                                                         \
    if (multi)                                                                                 \
      hipLaunchKernelGGL((gemv_down_kernel<NCP, true>), grid, block, lds, st, s.d, s.f, s.k,  \
                         s.E, w.down_q, w.down_s, idx, gate, h32, y);                          \
    else                                                                                       \
      hipLaunchKernelGGL((gemv_down_kernel<NCP, false>), grid, block, lds, st, s.d, s.f, s.k, \
                         s.E, w.down_q, w.down_s, idx, gate, h32, y);                          \
  } while (0)
  switch (ncp) {
    case 1: K3_DOWN(1); break;
    case 2: K3_DOWN(2); break;
    default: K3_DOWN(4); break;
  }
#undef K3_DOWN
  return hipGetLastError();
}

}  // namespace k3
