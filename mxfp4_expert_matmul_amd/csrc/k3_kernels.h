// Host-side launchers of the k3moe kernels (internal to the library).
// Every launcher enqueues on `stream` and returns the launch status; callers
// have validated all sizes and pointers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstddef>

namespace k3 {

// Prefill grouped GEMM tile: tokens (sorted pairs) per tile.
constexpr int kTileM = 96;
// Pairs per block of the grouping step.
constexpr int kGroupChunk = 256;
// Largest T served by the GEMV (decode) expert path.
constexpr int kGemvMaxT = 4;
// Largest T served by the GEMV router.
constexpr int kRouterGemvMaxT = 8;

struct Shape {
  int d, E, k, f;
};

struct ExpertWeights {
  const uint8_t *gate_q, *gate_s, *up_q, *up_s, *down_q, *down_s;
};

// layout.hip
size_t tiled_scale_bytes(int n, int R, int K);
hipError_t launch_pack(const uint8_t* codes, const uint8_t* scales, int n, int R, int K,
                       uint8_t* tcodes, uint8_t* tscales, hipStream_t st);

// router_topk.hip
hipError_t launch_router_logits(const uint16_t* x, int T, const Shape& s, const float* wr,
                                const uint16_t* wr3, const float* bias, float* logits,
                                hipStream_t st);
// three-term bf16 split of the router weights, w3 = [hi | mid | lo] each [E][d]
hipError_t launch_router_split(const float* wr, int E, int d, uint16_t* w3, hipStream_t st);
// sel_bias != NULL: the selection-only bias (ranks logits + sel_bias, gates
// from the logits alone)
hipError_t launch_topk(const float* logits, int T, const Shape& s, const float* sel_bias,
                       int32_t* idx, float* gate, hipStream_t st);

// group.hip
hipError_t launch_group(const int32_t* idx, int T, const Shape& s, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* bhist, int32_t* tiles,
                        int32_t* ntiles, hipStream_t st);

// gemv.hip (decode path, T <= kGemvMaxT)
// logits != NULL: each pair's expert comes from a top-k selection of its
// token's logits inside the kernel, which also writes idx and gate; else idx
// is the routing (gate unused)
hipError_t launch_gemv_gateup(const uint16_t* x, int T, const Shape& s, const ExpertWeights& w,
                              const float* logits, const float* sel_bias, int32_t* idx,
                              float* gate, float* h32, hipStream_t st);
hipError_t launch_gemv_down(int T, const Shape& s, const ExpertWeights& w, const int32_t* idx,
                            const float* gate, const float* h32, float* y, hipStream_t st);
// once per handle: raise the dynamic LDS limits the decode kernels of shape s need
hipError_t prepare_gemv(const Shape& s);
// the same for every decode kernel instantiation (no shape needed)
hipError_t prepare_gemv_all();

// gemm.hip (prefill path)
hipError_t launch_quant_x(const uint16_t* x, int T, int d, uint8_t* xq, uint8_t* xs,
                          hipStream_t st);
hipError_t launch_gemm_gateup(int T, const Shape& s, const ExpertWeights& w, const uint8_t* xq,
                              const uint8_t* xs, const int32_t* offsets, const int32_t* perm,
                              const int32_t* tiles, const int32_t* ntiles, int max_tiles,
                              uint8_t* hq, uint8_t* hs, hipStream_t st);
hipError_t launch_gemm_down(int T, const Shape& s, const ExpertWeights& w, const int32_t* offsets,
                            const int32_t* perm, const int32_t* tiles, const int32_t* ntiles,
                            int max_tiles, const uint8_t* hq, const uint8_t* hs, uint8_t* slots,
                            hipStream_t st);
hipError_t launch_combine(const uint8_t* slots, const int32_t* idx, const float* gate, int T,
                          const Shape& s, float* y, hipStream_t st);

}  // namespace k3
