// Device-side fill of the integer input streams of the synthetic MoE layer
// workloads, bit-identical to synth/__init__.py (numpy):
//   mix64 = SplitMix64 output finaliser, draw(i) = mix64(key + i) with
//   key = mix64(seed ^ (stream << 56)) computed by the caller;
//   codes:  byte b of a tensor = byte (b % 8) of draw(b / 8) (little endian)
//   scales: byte i = 123 + draw(i) % 5
// Input generation only: none of the layer's arithmetic lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void fill_codes_kernel(uint64_t* __restrict__ dst, uint64_t nwords, uint64_t key) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords;
       i += (uint64_t)gridDim.x * blockDim.x)
    dst[i] = mix64(key + i);
}

__global__ void fill_scales_kernel(uint8_t* __restrict__ dst, uint64_t n, uint64_t key) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    dst[i] = (uint8_t)(123u + (uint32_t)(mix64(key + i) % 5ull));
}

// Tiled layout (16-row x 128-column tiles, see the layer library's header):
// each thread writes one 16-byte lane chunk, which is 16 consecutive bytes of
// the row-major tensor, i.e. two draws.
__global__ void fill_codes_tiled_kernel(uint8_t* __restrict__ dst, uint64_t nchunks, int R, int K,
                                        uint64_t key) {
  const int KT = K / 128, RT = R / 16;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nchunks;
       i += (uint64_t)gridDim.x * blockDim.x) {
    const int l = (int)(i & 63);
    const uint64_t t = i >> 6;
    const int kt = (int)(t % KT);
    const uint64_t mrt = t / KT;
    const int rt = (int)(mrt % RT);
    const uint64_t m = mrt / RT;
    const uint64_t row = m * R + 16 * rt + (l & 15);
    const uint64_t c0 = row * (uint64_t)(K / 2) + 64 * kt + 16 * (l >> 4);  // multiple of 16
    uint64_t* d = reinterpret_cast<uint64_t*>(dst + 16 * i);
    d[0] = mix64(key + c0 / 8);
    d[1] = mix64(key + c0 / 8 + 1);
  }
}

__global__ void fill_scales_tiled_kernel(uint8_t* __restrict__ dst, uint64_t nwords, int R, int K,
                                         uint64_t key) {
  const int KT = K / 128, RT = R / 16, KG = (KT + 3) / 4, NB = K / 32;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords;
       i += (uint64_t)gridDim.x * blockDim.x) {
    const int l = (int)(i & 63);
    const uint64_t grp = i >> 6;
    const int kg = (int)(grp % KG);
    const uint64_t mrt = grp / KG;
    const int rt = (int)(mrt % RT);
    const uint64_t m = mrt / RT;
    const uint64_t row = m * R + 16 * rt + (l & 15);
    uint32_t w = 0;
    for (int j = 0; j < 4; ++j) {
      const int kt = 4 * kg + j;
      uint32_t b = 127u;
      if (kt < KT) b = 123u + (uint32_t)(mix64(key + row * NB + 4 * kt + (l >> 4)) % 5ull);
      w |= b << (8 * j);
    }
    reinterpret_cast<uint32_t*>(dst)[i] = w;
  }
}

}  // namespace

extern "C" {

// Fill n stacked R x K code matrices in the tiled layout.
int k3synth_fill_codes_tiled(void* dst, int n, int R, int K, uint64_t key, void* stream) {
  if (!dst || n <= 0 || R % 16 != 0 || K % 128 != 0) return -1;
  const uint64_t nchunks = (uint64_t)n * (R / 16) * (K / 128) * 64;
  hipLaunchKernelGGL(fill_codes_tiled_kernel, dim3(8192), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)dst, nchunks, R, K, key);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Fill the tiled scales of n stacked R x K matrices.
int k3synth_fill_scales_tiled(void* dst, int n, int R, int K, uint64_t key, void* stream) {
  if (!dst || n <= 0 || R % 16 != 0 || K % 128 != 0) return -1;
  const uint64_t nwords = (uint64_t)n * (R / 16) * ((K / 128 + 3) / 4) * 64;
  hipLaunchKernelGGL(fill_scales_tiled_kernel, dim3(8192), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)dst, nwords, R, K, key);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}


// Fill a whole code tensor of nbytes (multiple of 8, dst 8-byte aligned).
int k3synth_fill_codes(void* dst, uint64_t nbytes, uint64_t key, void* stream) {
  if (!dst || (nbytes % 8) != 0 || (reinterpret_cast<uintptr_t>(dst) % 8) != 0) return -1;
  if (nbytes == 0) return 0;
  hipLaunchKernelGGL(fill_codes_kernel, dim3(8192), dim3(256), 0, (hipStream_t)stream,
                     (uint64_t*)dst, nbytes / 8, key);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Fill a whole scale tensor of n bytes.
int k3synth_fill_scales(void* dst, uint64_t n, uint64_t key, void* stream) {
  if (!dst) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(fill_scales_kernel, dim3(8192), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)dst, n, key);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
