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

// cache_plan.hip (device-planned expert cache)
// Residency tables of an HBM arena of S expert slots for E experts, in device
// memory; the same fields as the host planner's (lru.h).
enum CacheCounter : int {
  kCtrStamp,      // counts every planned forward and prefetch
  kCtrLastFwd,    // stamp of the last planned forward (0: none)
  kCtrCalls,      // planned forwards
  kCtrHits,       // distinct experts found resident (raw: prefetched ones included)
  kCtrMisses,     // distinct experts copied in by forwards
  kCtrPfHits,     // hits on experts a prefetch brought in and no forward had used
  kCtrPrefetched, // experts copied in by prefetches
  kCtrPfRefused,  // prefetches refused for want of eligible slots
  kCtrIgnored,    // prefetch ids outside [0, E), skipped
  kCacheCounters = 16
};
struct CacheTables {
  int32_t* slot_of;     // [E] slot holding expert e, or -1
  int32_t* expert_in;   // [S] expert in slot s, or -1
  int64_t* last_use;    // [S] stamp of the last call that used slot s (0: never)
  int64_t* fwd_use;     // [S] stamp of the last forward that used slot s
  int32_t* pre;         // [S] 1: brought in by a prefetch, not used by a forward since
  int64_t* ctr;         // [kCacheCounters]
  int32_t* fwd_copies;  // [1 + 2 S] the last forward plan's copies: count, (expert, slot)...
  int32_t* pf_copies;   // [1 + 2 S] the last prefetch plan's copies
};
constexpr int kCacheTensors = 6;  // gate codes, gate scales, up codes, up scales, down codes, down scales
constexpr int kFillChunk = 65536;  // bytes of one expert per fill work item
// fill workgroups: they stride over the work items; 64 keep about 2 MB of
// PCIe reads in flight, which the link needs, and leave the other CUs to the
// expert kernels a prefetch overlaps
constexpr int kFillGrid = 64;
struct FillPlan {
  const uint8_t* src[kCacheTensors];  // device-visible pointers to the pinned host tensors
  uint8_t* dst[kCacheTensors];        // the arena's tensors
  uint64_t bytes[kCacheTensors];      // one expert's bytes of each tensor (multiples of 256)
  uint64_t total;                     // their sum
};
size_t cache_plan_forward_lds(int P, int E, int S);
size_t cache_plan_prefetch_lds(int E, int S);
// once per cache: raise the dynamic LDS limits of the two plan kernels
hipError_t prepare_cache_plan(int P, int E, int S);
// routes (top k of logits [T][E], selection-only bias sel_bias or NULL) and
// plans a forward: writes idx and gate [T][k] (and user_idx / user_gate when
// not NULL), the renamed selection sidx and the copy list; T k <= S
hipError_t launch_cache_plan_forward(const float* logits, int T, int k, const float* sel_bias,
                                     int E, int S, const CacheTables& tb, int32_t* idx,
                                     float* gate, int32_t* user_idx, float* user_gate,
                                     int32_t* sidx, hipStream_t st);
hipError_t launch_cache_plan_prefetch(const int32_t* experts, int n, int E, int S,
                                      const CacheTables& tb, hipStream_t st);
hipError_t launch_cache_fill(const int32_t* copies, int max_copies, int E, int S,
                             const FillPlan& fp, hipStream_t st);

}  // namespace k3
