// Device-side helpers shared by the k3moe HIP kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace k3 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// E8M0 scale byte -> fp32 value 2^(b-127); 0 -> 2^-127 (subnormal); 255 -> NaN
// (OCP Microscaling v1.0, E8M0).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  uint32_t u = b << 23;               // selects, not branches
  u = (b == 0u) ? 0x00400000u : u;
  u = (b == 255u) ? 0x7fc00000u : u;
  return __uint_as_float(u);
}

// Butterfly sum over the 64 lanes of a wave; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Sum over the 64 lanes through DPP (register-to-register, no LDS): quad
// swaps, half-row and row mirrors give every lane its 16-lane row's sum, row
// broadcasts of lanes 15 and 31 carry the rows forward; lane 63 holds the
// total, which every lane then reads.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf,
                                                        false));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = dpp_add<0xB1, 0xf>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xf>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xf>(v);  // row_half_mirror
  v = dpp_add<0x140, 0xf>(v);  // row_mirror
  v = dpp_add<0x142, 0xa>(v);  // row_bcast15 into rows 1 and 3
  v = dpp_add<0x143, 0xc>(v);  // row_bcast31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// SiLU(z) = z / (1 + e^-z), written so that large |z| neither overflows to
// NaN nor loses the sign: e^-z -> inf gives z / inf = -0.
__device__ __forceinline__ float silu_f32(float z) {
  return z / (1.0f + __expf(-z));
}

// Unbiased exponent of a finite non-zero fp32 magnitude (floor(log2 |a|)),
// subnormals included.
__device__ __forceinline__ int ilog2_f32(float a) {
  uint32_t u = __float_as_uint(a) & 0x7fffffffu;
  int e = (int)(u >> 23);
  if (e != 0) return e - 127;
  return -127 - (__clz(u) - 9);  // subnormal: leading mantissa bit position
}

// Round an fp32 value to the nearest OCP E4M3 value (ties to even), for
// |a| < 464 (no saturation needed). Returns the rounded value as fp32.
__device__ __forceinline__ float round_e4m3(float a) {
  float m = fabsf(a);
  if (m == 0.0f) return a;
  int e = ilog2_f32(m);
  if (e < -6) e = -6;  // subnormal spacing 2^-9
  float ulp = __uint_as_float((uint32_t)(e - 3 + 127) << 23);
  return rintf(a / ulp) * ulp;
}

// E8M0 byte of the scale 2^(floor(log2 amax) - 7) that maps the block max
// into [128, 256) of E4M3 (no clamping at 448); amax == 0 gives 127.
__device__ __forceinline__ uint32_t e4m3_block_scale_byte(float amax) {
  if (!(amax > 0.0f)) return 127u;
  int b = ilog2_f32(amax) - 7 + 127;
  if (b < 0) b = 0;
  if (b > 254) b = 254;
  return (uint32_t)b;
}

// Pack 4 fp32 values that are exactly representable in E4M3 into 4 bytes
// (hardware convert, round-to-nearest-even, scale 1).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  v2s w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, 1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, 1.0f, true);
  return __builtin_bit_cast(uint32_t, w);
}

}  // namespace k3
