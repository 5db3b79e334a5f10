// Tiled MXFP4 layout read by every expert kernel, and the entry point that
// builds it from the row-major layout.
//
// A matrix of R rows and K columns (R % 16 == 0, K % 128 == 0) is cut into
// 16-row x 128-column tiles, (rt, kt) with RT = R/16, KT = K/128.
//   codes : tile (rt, kt) = 1024 bytes at ((rt*KT + kt) * 1024); inside it,
//           lane l = r + 16 g (r = row % 16, g = (col % 128) / 32) owns bytes
//           [16 l, 16 l + 16) = the 32-element MX block of row 16 rt + r,
//           columns 128 kt + 32 g .. +31, element 2i in the low nibble of
//           byte i (the same bytes as in the row-major layout);
//   scales: for KG = ceil(KT/4) groups of four K tiles, group (rt, kg) = 256
//           bytes at ((rt*KG + kg) * 256); lane l owns bytes [4 l, 4 l + 4),
//           byte j = the E8M0 scale of that lane's block in tile kt = 4 kg + j
//           (127 where 4 kg + j >= KT).
// One 1024-byte tile is exactly the A operand of one 16x16x128 MX MFMA (lane
// l holds row l % 16, K block l / 16), so a wave loads it with one fully
// coalesced 16-byte-per-lane instruction, and one 4-byte scale load serves
// four K steps. Stacked matrices (experts) follow each other.
#include "k3_device.h"
#include "k3_kernels.h"

namespace k3 {

// One thread per 16-byte lane chunk of the tiled codes.
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ src,
                                                         int R, int K, size_t nchunks,
                                                         uint8_t* __restrict__ dst) {
  const int KT = K / 128, RT = R / 16;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nchunks;
       i += (size_t)gridDim.x * 256) {
    const int l = (int)(i & 63);
    const size_t t = i >> 6;  // global tile index (matrix, rt, kt)
    const int kt = (int)(t % KT);
    const size_t mrt = t / KT;  // matrix * RT + rt
    const int rt = (int)(mrt % RT);
    const size_t m = mrt / RT;
    const size_t row = m * R + 16 * rt + (l & 15);
    const uint4 v =
        *reinterpret_cast<const uint4*>(src + row * (size_t)(K / 2) + 64 * kt + 16 * (l >> 4));
    *reinterpret_cast<uint4*>(dst + 16 * i) = v;
  }
}

// One thread per 4-byte lane word of the tiled scales.
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ src,
                                                          int R, int K, size_t nwords,
                                                          uint8_t* __restrict__ dst) {
  const int KT = K / 128, RT = R / 16, KG = (KT + 3) / 4, NB = K / 32;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nwords;
       i += (size_t)gridDim.x * 256) {
    const int l = (int)(i & 63);
    const size_t grp = i >> 6;  // (matrix, rt, kg)
    const int kg = (int)(grp % KG);
    const size_t mrt = grp / KG;
    const int rt = (int)(mrt % RT);
    const size_t m = mrt / RT;
    const size_t row = m * R + 16 * rt + (l & 15);
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kt = 4 * kg + j;
      const uint32_t b = (kt < KT) ? src[row * NB + 4 * kt + (l >> 4)] : 127u;
      w |= b << (8 * j);
    }
    reinterpret_cast<uint32_t*>(dst)[i] = w;
  }
}

size_t tiled_scale_bytes(int n, int R, int K) {
  const int KT = K / 128, KG = (KT + 3) / 4;
  return (size_t)n * (R / 16) * KG * 256;
}

hipError_t launch_pack(const uint8_t* codes, const uint8_t* scales, int n, int R, int K,
                       uint8_t* tcodes, uint8_t* tscales, hipStream_t st) {
  const size_t nchunks = (size_t)n * (R / 16) * (K / 128) * 64;
  const size_t nwords = tiled_scale_bytes(n, R, K) / 4;
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)std::min<size_t>((nchunks + 255) / 256, 65536)),
                     dim3(256), 0, st, codes, R, K, nchunks, tcodes);
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)std::min<size_t>((nwords + 255) / 256, 65536)),
                     dim3(256), 0, st, scales, R, K, nwords, tscales);
  return hipGetLastError();
}

}  // namespace k3
