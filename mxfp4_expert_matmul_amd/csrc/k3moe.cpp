// Host side of the k3moe C ABI: argument checks, workspace planning and
// allocation, and dispatch of the router, grouping and expert kernels.
// The library never aborts, exits or prints; every failure is a status code.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "k3_kernels.h"
#include "k3moe.h"
#include "k3moe_internal.h"

using k3::Shape;

namespace {

constexpr size_t kAlign = 256;
// device staging of k3moe_pack_mxfp4_from_host: row-major matrices per chunk
constexpr size_t kPackStageBytes = (size_t)32 << 20;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Byte offsets of every workspace buffer for one config.
struct Plan {
  size_t logits, idx, gate, counts, offsets, perm, bhist, tiles, ntiles, xq, xs, hq, hs, h32,
      slots, wr3;
  size_t total;
  int max_tiles;
};

int check_config(const k3moe_config* c) {
  if (!c) return K3MOE_EINVAL;
  if ((c->flags & ~K3MOE_FLAG_BIAS_SELECT_ONLY) != 0u) return K3MOE_EINVAL;
  if (c->d_model <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->d_ff <= 0 ||
      c->max_tokens <= 0)
    return K3MOE_EINVAL;
  if (c->top_k > c->n_experts) return K3MOE_EINVAL;
  if (c->d_model % 32 != 0 || c->d_ff % 32 != 0) return K3MOE_EINVAL;  // whole MX blocks
  if (c->d_model % 128 != 0 || c->d_ff % 128 != 0) return K3MOE_EUNSUPPORTED;
  if (c->d_model > 8192 || c->d_ff > 4096) return K3MOE_EUNSUPPORTED;
  if (c->n_experts > 4096 || c->top_k > 64) return K3MOE_EUNSUPPORTED;
  if ((int64_t)c->max_tokens * c->top_k >= (int64_t)1 << 31) return K3MOE_EUNSUPPORTED;
  // the prefill kernels address one plane of the activation split (T x d) and
  // of the h split (T*k x f) with 32-bit byte offsets, and use offsets from
  // 2^31 - 2^16 up as "read nothing"
  if ((int64_t)c->max_tokens * c->d_model > (int64_t)1 << 30 ||
      (int64_t)c->max_tokens * c->top_k * c->d_ff > (int64_t)1 << 30)
    return K3MOE_EUNSUPPORTED;
  return K3MOE_OK;
}

Plan make_plan(const k3moe_config* c) {
  const size_t T = (size_t)c->max_tokens, E = (size_t)c->n_experts, k = (size_t)c->top_k;
  const size_t d = (size_t)c->d_model, f = (size_t)c->d_ff;
  const size_t P = T * k;
  const size_t NB = (P + k3::kGroupChunk - 1) / k3::kGroupChunk;
  const size_t tiles = (P + k3::kTileM - 1) / k3::kTileM + std::min(E, P);
  const size_t tg = std::min(T, (size_t)k3::kGemvMaxT);
  Plan p{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align_up(bytes);
    return at;
  };
  p.logits = take(T * E * 4);
  p.idx = take(P * 4);
  p.gate = take(P * 4);
  p.counts = take(E * 4);
  p.offsets = take((E + 1) * 4);
  p.perm = take(P * 4);
  p.bhist = take(NB * E * 4);
  p.tiles = take(tiles * 2 * 4);
  p.ntiles = take(4);
  p.xq = take(2 * T * d);
  p.xs = take(2 * T * (d / 32));
  p.hq = take(2 * P * f);
  p.hs = take(2 * P * (f / 32));
  p.h32 = take(tg * k * f * 4);
  p.slots = take(P * d * 3);  // 24-bit floats
  p.wr3 = take(3 * E * d * 2);
  p.total = o;
  p.max_tiles = (int)tiles;
  return p;
}

// Restores the caller's current device on scope exit.
struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) return;
    ok = (prev == dev) || (hipSetDevice(dev) == hipSuccess);
  }
  ~DeviceGuard() {
    if (ok && prev >= 0) (void)hipSetDevice(prev);
  }
};

}  // namespace

struct k3moe {
  k3moe_config cfg;
  k3moe_weights w;
  int device;
  Plan plan;
  uint8_t* ws;
  // typed views into ws
  float* logits;
  int32_t* idx;
  float* gate;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* bhist;
  int32_t* tiles;
  int32_t* ntiles;
  uint8_t* xq;
  uint8_t* xs;
  uint8_t* hq;
  uint8_t* hs;
  float* h32;  // decode: SwiGLU output per pair
  uint8_t* slots;
  uint16_t* wr3;  // router weights as three bf16 terms, derived at create
  // stage timing (k3moe_profile_begin / k3moe_profile_end)
  bool prof_on;
  int prof_cap;
  uint32_t prof_mask;  // stages timed (bit i: stage i)
  int prof_n[K3MOE_NUM_STAGES];
  std::vector<hipEvent_t> prof_ev[K3MOE_NUM_STAGES];  // 2 per recorded launch
  // a second stream (default priority) on which the whole-layer call splits x
  // for the prefill GEMM while the router runs on the caller's stream
  hipStream_t side;
  hipEvent_t ev_fork, ev_join;
};

namespace {

void profile_release(k3moe* h) {
  for (int i = 0; i < K3MOE_NUM_STAGES; ++i) {
    for (hipEvent_t ev : h->prof_ev[i]) (void)hipEventDestroy(ev);
    h->prof_ev[i].clear();
    h->prof_n[i] = 0;
  }
  h->prof_on = false;
  h->prof_cap = 0;
  h->prof_mask = 0;
}

// The router bias as the logit kernels see it (added to every logit) and as
// the top-k sees it (added only to rank: the selection-only bias).
const float* logit_bias(const k3moe_config& c, const float* b) {
  return (c.flags & K3MOE_FLAG_BIAS_SELECT_ONLY) ? nullptr : b;
}
const float* select_bias(const k3moe_config& c, const float* b) {
  return (c.flags & K3MOE_FLAG_BIAS_SELECT_ONLY) ? b : nullptr;
}

Shape shape_of(const k3moe* h) {
  return Shape{h->cfg.d_model, h->cfg.n_experts, h->cfg.top_k, h->cfg.d_ff};
}

k3::ExpertWeights experts_of(const k3moe* h) {
  return k3::ExpertWeights{h->w.gate_q, h->w.gate_s, h->w.up_q, h->w.up_s, h->w.down_q, h->w.down_s};
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? K3MOE_OK : K3MOE_EHIP; }

// Runs one stage's launch, bracketed by HIP events on the same stream when
// stage timing is on.
template <class F>
hipError_t stage(k3moe* h, int id, hipStream_t st, F&& launch) {
  const bool rec = h->prof_on && ((h->prof_mask >> id) & 1u) && h->prof_n[id] < h->prof_cap;
  if (rec) {
    hipError_t e = hipEventRecord(h->prof_ev[id][2 * h->prof_n[id]], st);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch();
  if (e != hipSuccess) return e;
  if (rec) {
    e = hipEventRecord(h->prof_ev[id][2 * h->prof_n[id] + 1], st);
    if (e != hipSuccess) return e;
    h->prof_n[id]++;
  }
  return hipSuccess;
}

// Router logits, then (with_topk) the top-k selection into idx and gate.
int run_router(k3moe* h, const uint16_t* x, int T, float* logits, int32_t* idx, float* gate,
               hipStream_t st, bool with_topk = true) {
  const Shape s = shape_of(h);
  hipError_t e = stage(h, K3MOE_STAGE_ROUTER_LOGITS, st, [&] {
    return k3::launch_router_logits(x, T, s, h->w.router_w, h->wr3,
                                    logit_bias(h->cfg, h->w.router_b), logits, st);
  });
  if (e != hipSuccess) return K3MOE_EHIP;
  if (!with_topk) return K3MOE_OK;
  e = stage(h, K3MOE_STAGE_TOPK, st, [&] {
    return k3::launch_topk(logits, T, s, select_bias(h->cfg, h->w.router_b), idx, gate, st);
  });
  return hip_status(e);
}

// The expert FFNs and the combine. With `logits` (GEMV path only) the
// gate/up GEMV selects each token's experts itself and writes idx and gate;
// otherwise idx and gate are the routing and are only read.
int run_experts(k3moe* h, const uint16_t* x, int T, int32_t* idx, float* gate, float* y,
                hipStream_t st, const float* logits = nullptr, bool x_split_on_side = false) {
  const Shape s = shape_of(h);
  const k3::ExpertWeights w = experts_of(h);
  hipError_t e;
  if (T <= k3::kGemvMaxT) {
    e = stage(h, K3MOE_STAGE_GATEUP, st, [&] {
      return k3::launch_gemv_gateup(x, T, s, w, logits, select_bias(h->cfg, h->w.router_b), idx,
                                    gate, h->h32, st);
    });
    if (e != hipSuccess) return K3MOE_EHIP;
    e = stage(h, K3MOE_STAGE_DOWN, st,
              [&] { return k3::launch_gemv_down(T, s, w, idx, gate, h->h32, y, st); });
    return hip_status(e);
  }
  e = stage(h, K3MOE_STAGE_GROUP, st, [&] {
    return k3::launch_group(idx, T, s, h->counts, h->offsets, h->perm, h->bhist, h->tiles,
                            h->ntiles, st);
  });
  if (e != hipSuccess) return K3MOE_EHIP;
  if (x_split_on_side) {
    // the split of x was enqueued on the side stream before the router
    e = hipStreamWaitEvent(st, h->ev_join, 0);
  } else {
    e = stage(h, K3MOE_STAGE_QUANT_X, st,
              [&] { return k3::launch_quant_x(x, T, s.d, h->xq, h->xs, st); });
  }
  if (e != hipSuccess) return K3MOE_EHIP;
  // the tile bound for this call's T (never above the workspace's)
  const size_t P = (size_t)T * s.k;
  const int max_tiles = (int)((P + k3::kTileM - 1) / k3::kTileM + std::min((size_t)s.E, P));
  e = stage(h, K3MOE_STAGE_GATEUP, st, [&] {
    return k3::launch_gemm_gateup(T, s, w, h->xq, h->xs, h->offsets, h->perm, h->tiles,
                                  h->ntiles, max_tiles, h->hq, h->hs, st);
  });
  if (e != hipSuccess) return K3MOE_EHIP;
  e = stage(h, K3MOE_STAGE_DOWN, st, [&] {
    return k3::launch_gemm_down(T, s, w, h->offsets, h->perm, h->tiles, h->ntiles, max_tiles,
                                h->hq, h->hs, h->slots, st);
  });
  if (e != hipSuccess) return K3MOE_EHIP;
  e = stage(h, K3MOE_STAGE_COMBINE, st,
            [&] { return k3::launch_combine(h->slots, idx, gate, T, s, y, st); });
  return hip_status(e);
}

int check_tokens(const k3moe* h, int32_t T) {
  if (!h) return K3MOE_EINVAL;
  if (T < 0 || T > h->cfg.max_tokens) return K3MOE_EINVAL;
  return K3MOE_OK;
}

// ------------------------------------------------------ no-allocation decode
// k3moe_layer_forward_noalloc serves callers that cannot allocate (code under
// HIP graph capture, serving loops, harnesses that forbid hipMalloc). It runs
// the decode path (T <= kGemvMaxT: router GEMV, gate/up GEMV with the top-k
// fused, down GEMV with the combine fused) with its scratch -- the logits,
// the routing when the caller passes none, and the SwiGLU output h -- in this
// file-scope device array. Each device holds its own copy for the life of
// the process; calls on one device share it (overlapping calls race).
constexpr size_t kScratchBytes = (size_t)2 << 20;  // 2 MiB
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The array's device address, taken once per device with that device
// current (host code never passes the array's own name to a kernel: on the
// host it names a stand-in, not device memory).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

hipError_t scratch_of_device(int dev, uint8_t** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    // the decode kernels' dynamic LDS limits, once per device
    e = k3::prepare_gemv_all();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<uint8_t*>(g_scratch_ptr[dev]);
  return hipSuccess;
}

// Scratch bytes a decode call of T tokens needs (logits, h, and idx/gate
// when the caller passes none), each slice 256-byte aligned.
size_t noalloc_scratch_bytes(const k3moe_config* c, int T, bool own_routing) {
  const size_t P = (size_t)T * c->top_k;
  size_t n = align_up((size_t)T * c->n_experts * 4) + align_up(P * c->d_ff * 4);
  if (own_routing) n += 2 * align_up(P * 4);
  return n;
}

}  // namespace

int k3::route_logits(k3moe* h, const void* x, int32_t T, float* logits, hipStream_t st) {
  int rc = check_tokens(h, T);
  if (rc != K3MOE_OK) return rc;
  if (T == 0) return K3MOE_OK;
  if (!x || !logits || !aligned(x, 16) || !aligned(logits, 4)) return K3MOE_EINVAL;
  DeviceGuard guard(h->device);
  if (!guard.ok) return K3MOE_EHIP;
  return run_router(h, static_cast<const uint16_t*>(x), T, logits, nullptr, nullptr, st,
                    /*with_topk=*/false);
}

extern "C" {

const char* k3moe_status_str(int status) {
  switch (status) {
    case K3MOE_OK: return "ok";
    case K3MOE_EINVAL: return "invalid argument";
    case K3MOE_ENOMEM: return "not enough device memory for the workspace";
    case K3MOE_EHIP: return "HIP runtime or kernel launch failure";
    case K3MOE_EUNSUPPORTED: return "configuration outside what the library supports";
    default: return "unknown status";
  }
}

int64_t k3moe_tiled_scale_bytes(int32_t n, int32_t R, int32_t K) {
  if (n <= 0 || R <= 0 || K <= 0 || R % 16 != 0 || K % 128 != 0) return 0;
  return (int64_t)k3::tiled_scale_bytes(n, R, K);
}

int k3moe_pack_mxfp4(const uint8_t* codes, const uint8_t* scales, int32_t n, int32_t R, int32_t K,
                     uint8_t* tiled_codes, uint8_t* tiled_scales, void* stream) {
  if (!codes || !scales || !tiled_codes || !tiled_scales) return K3MOE_EINVAL;
  if (n <= 0 || R <= 0 || K <= 0 || R % 16 != 0 || K % 128 != 0) return K3MOE_EINVAL;
  const void* ps[] = {codes, scales, tiled_codes, tiled_scales};
  for (const void* p : ps)
    if (!aligned(p, 16)) return K3MOE_EINVAL;
  return hip_status(k3::launch_pack(codes, scales, n, R, K, tiled_codes, tiled_scales,
                                    static_cast<hipStream_t>(stream)));
}

int k3moe_pack_mxfp4_from_host(const uint8_t* codes, const uint8_t* scales, int32_t n, int32_t R,
                               int32_t K, uint8_t* tiled_codes, uint8_t* tiled_scales,
                               void* stream) {
  if (!codes || !scales || !tiled_codes || !tiled_scales) return K3MOE_EINVAL;
  if (n <= 0 || R <= 0 || K <= 0 || R % 16 != 0 || K % 128 != 0) return K3MOE_EINVAL;
  if (!aligned(tiled_codes, 16) || !aligned(tiled_scales, 16)) return K3MOE_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t cb = (size_t)R * K / 2, sb = (size_t)R * (K / 32);  // one matrix, row-major
  const size_t tb = k3::tiled_scale_bytes(1, R, K);                 // its tiled scales
  // matrices per chunk: as many as fit the staging bytes, at least one
  const size_t per = align_up(cb) + align_up(sb);
  const size_t m = std::max<size_t>(1, std::min<size_t>((size_t)n, kPackStageBytes / per));
  const size_t stage_bytes = align_up(m * cb) + align_up(m * sb);
  size_t free_b = 0, total_b = 0;
  if (hipMemGetInfo(&free_b, &total_b) != hipSuccess) {
    (void)hipGetLastError();
    return K3MOE_EHIP;
  }
  if (stage_bytes > free_b) return K3MOE_ENOMEM;
  void* stage = nullptr;
  if (hipMalloc(&stage, stage_bytes) != hipSuccess || !stage) {
    (void)hipGetLastError();
    return K3MOE_ENOMEM;
  }
  uint8_t* sc = static_cast<uint8_t*>(stage);
  uint8_t* ss = sc + align_up(m * cb);
  // chunk by chunk on one stream: its copy lands after the previous chunk's
  // pack has read the staging buffer (stream order)
  hipError_t e = hipSuccess;
  for (size_t i0 = 0; i0 < (size_t)n && e == hipSuccess; i0 += m) {
    const size_t cnt = std::min(m, (size_t)n - i0);
    e = hipMemcpyAsync(sc, codes + i0 * cb, cnt * cb, hipMemcpyHostToDevice, st);
    if (e == hipSuccess)
      e = hipMemcpyAsync(ss, scales + i0 * sb, cnt * sb, hipMemcpyHostToDevice, st);
    if (e == hipSuccess)
      e = k3::launch_pack(sc, ss, (int)cnt, R, K, tiled_codes + i0 * cb, tiled_scales + i0 * tb, st);
  }
  const hipError_t es = hipStreamSynchronize(st);  // the staging buffer is free after this
  (void)hipFree(stage);
  if (e != hipSuccess || es != hipSuccess) {
    (void)hipGetLastError();
    return K3MOE_EHIP;
  }
  return K3MOE_OK;
}

int64_t k3moe_workspace_bytes(const k3moe_config* cfg) {
  int rc = check_config(cfg);
  if (rc != K3MOE_OK) return rc;
  return (int64_t)make_plan(cfg).total;
}

int k3moe_create(const k3moe_config* cfg, const k3moe_weights* w, int device, k3moe** out) {
  if (out) *out = nullptr;
  if (!out || !w) return K3MOE_EINVAL;
  int rc = check_config(cfg);
  if (rc != K3MOE_OK) return rc;
  const void* req[] = {w->router_w, w->gate_q, w->gate_s, w->up_q, w->up_s, w->down_q, w->down_s};
  for (const void* p : req)
    if (!p || !aligned(p, 16)) return K3MOE_EINVAL;
  if (w->router_b && !aligned(w->router_b, 16)) return K3MOE_EINVAL;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) return K3MOE_EHIP;
  if (device < 0 || device >= ndev) return K3MOE_EINVAL;
  DeviceGuard guard(device);
  if (!guard.ok) return K3MOE_EHIP;
  const Plan plan = make_plan(cfg);
  size_t free_b = 0, total_b = 0;
  if (hipMemGetInfo(&free_b, &total_b) != hipSuccess) return K3MOE_EHIP;
  if (plan.total > free_b) return K3MOE_ENOMEM;  // refuse before allocating
  k3moe* h = new (std::nothrow) k3moe();
  if (!h) return K3MOE_ENOMEM;
  h->cfg = *cfg;
  h->w = *w;
  h->device = device;
  h->plan = plan;
  void* base = nullptr;
  if (hipMalloc(&base, plan.total) != hipSuccess || !base) {
    (void)hipGetLastError();  // clear the sticky allocation error
    delete h;
    return K3MOE_ENOMEM;
  }
  h->ws = static_cast<uint8_t*>(base);
  h->logits = reinterpret_cast<float*>(h->ws + plan.logits);
  h->idx = reinterpret_cast<int32_t*>(h->ws + plan.idx);
  h->gate = reinterpret_cast<float*>(h->ws + plan.gate);
  h->counts = reinterpret_cast<int32_t*>(h->ws + plan.counts);
  h->offsets = reinterpret_cast<int32_t*>(h->ws + plan.offsets);
  h->perm = reinterpret_cast<int32_t*>(h->ws + plan.perm);
  h->bhist = reinterpret_cast<int32_t*>(h->ws + plan.bhist);
  h->tiles = reinterpret_cast<int32_t*>(h->ws + plan.tiles);
  h->ntiles = reinterpret_cast<int32_t*>(h->ws + plan.ntiles);
  h->xq = h->ws + plan.xq;
  h->xs = h->ws + plan.xs;
  h->hq = h->ws + plan.hq;
  h->hs = h->ws + plan.hs;
  h->h32 = reinterpret_cast<float*>(h->ws + plan.h32);
  h->slots = h->ws + plan.slots;
  h->wr3 = reinterpret_cast<uint16_t*>(h->ws + plan.wr3);
  if (k3::prepare_gemv(shape_of(h)) != hipSuccess ||
      k3::launch_router_split(w->router_w, cfg->n_experts, cfg->d_model, h->wr3, nullptr) !=
          hipSuccess ||
      hipStreamSynchronize(nullptr) != hipSuccess ||
      hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
    if (h->side) (void)hipStreamDestroy(h->side);
    (void)hipFree(h->ws);
    delete h;
    return K3MOE_EHIP;
  }
  *out = h;
  return K3MOE_OK;
}

void k3moe_destroy(k3moe* h) {
  if (!h) return;
  {
    DeviceGuard guard(h->device);
    if (guard.ok) {
      (void)hipDeviceSynchronize();
      profile_release(h);
      (void)hipEventDestroy(h->ev_join);
      (void)hipEventDestroy(h->ev_fork);
      (void)hipStreamDestroy(h->side);
      (void)hipFree(h->ws);
    }
  }
  delete h;
}

int k3moe_route(k3moe* h, const void* x, int32_t T, float* logits, int32_t* idx, float* gate,
                void* stream) {
  int rc = check_tokens(h, T);
  if (rc != K3MOE_OK) return rc;
  if (T == 0) return K3MOE_OK;
  if (!x || !idx || !gate || !aligned(x, 16) || !aligned(idx, 4) || !aligned(gate, 4))
    return K3MOE_EINVAL;
  if (logits && !aligned(logits, 4)) return K3MOE_EINVAL;
  DeviceGuard guard(h->device);
  if (!guard.ok) return K3MOE_EHIP;
  float* lg = logits ? logits : h->logits;
  return run_router(h, static_cast<const uint16_t*>(x), T, lg, idx, gate,
                    static_cast<hipStream_t>(stream));
}

int k3moe_group(k3moe* h, const int32_t* idx, int32_t T, int32_t* counts, int32_t* offsets,
                int32_t* perm, void* stream) {
  int rc = check_tokens(h, T);
  if (rc != K3MOE_OK) return rc;
  if (!counts || !offsets || (T > 0 && (!idx || !perm))) return K3MOE_EINVAL;
  if (!aligned(idx, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(perm, 4))
    return K3MOE_EINVAL;
  DeviceGuard guard(h->device);
  if (!guard.ok) return K3MOE_EHIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // T == 0 still writes zero counts and offsets
  return hip_status(stage(h, K3MOE_STAGE_GROUP, st, [&] {
    return k3::launch_group(idx, T, shape_of(h), counts, offsets, perm, h->bhist, h->tiles,
                            h->ntiles, st);
  }));
}

int k3moe_experts_forward(k3moe* h, const void* x, int32_t T, const int32_t* idx,
                          const float* gate, float* y, void* stream) {
  int rc = check_tokens(h, T);
  if (rc != K3MOE_OK) return rc;
  if (T == 0) return K3MOE_OK;
  if (!x || !idx || !gate || !y) return K3MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(idx, 4) || !aligned(gate, 4))
    return K3MOE_EINVAL;
  DeviceGuard guard(h->device);
  if (!guard.ok) return K3MOE_EHIP;
  // without logits run_experts only reads idx and gate
  return run_experts(h, static_cast<const uint16_t*>(x), T, const_cast<int32_t*>(idx),
                     const_cast<float*>(gate), y, static_cast<hipStream_t>(stream));
}

int k3moe_layer_forward(k3moe* h, const void* x, int32_t T, float* y, int32_t* topk_idx,
                        float* topk_gate, void* stream) {
  int rc = check_tokens(h, T);
  if (rc != K3MOE_OK) return rc;
  if (T == 0) return K3MOE_OK;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return K3MOE_EINVAL;
  if ((topk_idx && !aligned(topk_idx, 4)) || (topk_gate && !aligned(topk_gate, 4)))
    return K3MOE_EINVAL;
  DeviceGuard guard(h->device);
  if (!guard.ok) return K3MOE_EHIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* idx = topk_idx ? topk_idx : h->idx;
  float* gate = topk_gate ? topk_gate : h->gate;
  // few tokens: the gate/up GEMV does the top-k selection (one launch fewer)
  const bool fused_topk = T <= k3::kGemvMaxT;
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (!fused_topk) {
    // the split of x for the prefill GEMM needs only x: it runs on the side
    // stream, after everything already on the caller's stream, while the
    // router runs (the router leaves CUs idle at large T); the gate/up GEMM
    // waits for it
    const Shape s = shape_of(h);
    hipError_t e = hipEventRecord(h->ev_fork, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(h->side, h->ev_fork, 0);
    if (e == hipSuccess)
      e = stage(h, K3MOE_STAGE_QUANT_X, h->side,
                [&] { return k3::launch_quant_x(xb, T, s.d, h->xq, h->xs, h->side); });
    if (e == hipSuccess) e = hipEventRecord(h->ev_join, h->side);
    if (e != hipSuccess) return K3MOE_EHIP;
  }
  int rc2 = run_router(h, xb, T, h->logits, idx, gate, st, !fused_topk);
  if (rc2 != K3MOE_OK) {
    if (!fused_topk) (void)hipStreamWaitEvent(st, h->ev_join, 0);  // keep the side joined
    return rc2;
  }
  return run_experts(h, xb, T, idx, gate, y, st, fused_topk ? h->logits : nullptr, !fused_topk);
}

int k3moe_layer_forward_noalloc(const k3moe_config* cfg, const k3moe_weights* w, const void* x,
                                int32_t T, float* y, int32_t* topk_idx, float* topk_gate,
                                void* stream) {
  int rc = check_config(cfg);
  if (rc != K3MOE_OK) return rc;
  if (!w) return K3MOE_EINVAL;
  const void* req[] = {w->router_w, w->gate_q, w->gate_s, w->up_q, w->up_s, w->down_q, w->down_s};
  for (const void* p : req)
    if (!p || !aligned(p, 16)) return K3MOE_EINVAL;
  if (w->router_b && !aligned(w->router_b, 16)) return K3MOE_EINVAL;
  if (T < 0 || T > cfg->max_tokens) return K3MOE_EINVAL;
  if (T == 0) return K3MOE_OK;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return K3MOE_EINVAL;
  if ((topk_idx && !aligned(topk_idx, 4)) || (topk_gate && !aligned(topk_gate, 4)))
    return K3MOE_EINVAL;
  if ((topk_idx == nullptr) != (topk_gate == nullptr)) return K3MOE_EINVAL;
  // the decode path only, within the fixed scratch
  if (T > k3::kGemvMaxT) return K3MOE_EUNSUPPORTED;
  const bool own = topk_idx == nullptr;
  if (noalloc_scratch_bytes(cfg, T, own) > kScratchBytes) return K3MOE_EUNSUPPORTED;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return K3MOE_EHIP;
  if (dev >= kMaxDevices) return K3MOE_EUNSUPPORTED;
  uint8_t* base = nullptr;
  if (scratch_of_device(dev, &base) != hipSuccess) {
    (void)hipGetLastError();
    return K3MOE_EHIP;
  }
  const size_t P = (size_t)T * cfg->top_k;
  float* logits = reinterpret_cast<float*>(base);
  size_t o = align_up((size_t)T * cfg->n_experts * 4);
  float* h32 = reinterpret_cast<float*>(base + o);
  o += align_up(P * cfg->d_ff * 4);
  int32_t* idx = topk_idx;
  float* gate = topk_gate;
  if (own) {
    idx = reinterpret_cast<int32_t*>(base + o);
    o += align_up(P * 4);
    gate = reinterpret_cast<float*>(base + o);
  }
  const Shape s{cfg->d_model, cfg->n_experts, cfg->top_k, cfg->d_ff};
  const k3::ExpertWeights ew{w->gate_q, w->gate_s, w->up_q, w->up_s, w->down_q, w->down_s};
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  hipError_t e = k3::launch_router_logits(xb, T, s, w->router_w, nullptr,
                                          logit_bias(*cfg, w->router_b), logits, st);
  if (e == hipSuccess)
    e = k3::launch_gemv_gateup(xb, T, s, ew, logits, select_bias(*cfg, w->router_b), idx, gate,
                               h32, st);
  if (e == hipSuccess) e = k3::launch_gemv_down(T, s, ew, idx, gate, h32, y, st);
  return hip_status(e);
}


int k3moe_profile_begin(k3moe* h, int32_t max_calls) {
  return k3moe_profile_begin_stages(h, max_calls, (1u << K3MOE_NUM_STAGES) - 1u);
}

int k3moe_profile_begin_stages(k3moe* h, int32_t max_calls, uint32_t stage_mask) {
  if (!h || max_calls <= 0 || max_calls > (1 << 20)) return K3MOE_EINVAL;
  if (stage_mask == 0 || (stage_mask >> K3MOE_NUM_STAGES) != 0) return K3MOE_EINVAL;
  DeviceGuard guard(h->device);
  if (!guard.ok) return K3MOE_EHIP;
  profile_release(h);
  for (int i = 0; i < K3MOE_NUM_STAGES; ++i) {
    if (!((stage_mask >> i) & 1u)) continue;
    try {
      h->prof_ev[i].resize(2 * (size_t)max_calls, nullptr);
    } catch (...) {
      profile_release(h);
      return K3MOE_ENOMEM;
    }
    for (auto& ev : h->prof_ev[i]) {
      if (hipEventCreate(&ev) != hipSuccess) {
        ev = nullptr;
        profile_release(h);
        return K3MOE_EHIP;
      }
    }
  }
  h->prof_cap = max_calls;
  h->prof_mask = stage_mask;
  h->prof_on = true;
  return K3MOE_OK;
}

int k3moe_profile_end(k3moe* h, float* total_ms, int32_t* launches) {
  if (!h || !total_ms || !launches) return K3MOE_EINVAL;
  if (!h->prof_on) return K3MOE_EINVAL;
  DeviceGuard guard(h->device);
  if (!guard.ok) return K3MOE_EHIP;
  int rc = K3MOE_OK;
  for (int i = 0; i < K3MOE_NUM_STAGES; ++i) {
    double sum = 0.0;
    for (int n = 0; n < h->prof_n[i]; ++n) {
      float ms = 0.0f;
      if (hipEventSynchronize(h->prof_ev[i][2 * n + 1]) != hipSuccess ||
          hipEventElapsedTime(&ms, h->prof_ev[i][2 * n], h->prof_ev[i][2 * n + 1]) != hipSuccess) {
        rc = K3MOE_EHIP;
        continue;
      }
      sum += ms;
    }
    total_ms[i] = (float)sum;
    launches[i] = h->prof_n[i];
  }
  profile_release(h);
  return rc;
}

}  // extern "C"
