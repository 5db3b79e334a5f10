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

}  // namespace

extern "C" {

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
