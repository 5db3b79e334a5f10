// Expert cache for layers whose experts live in host memory: an HBM arena of
// n_slots experts, replaced least-recently-used, filled over PCIe as the
// routing asks for experts (the GPU counterpart of the pages' LRU expert
// cache in RAM in front of NVMe; ssnai.com decision guide and xugj520.cn run
// notes on raw versus true resident hits).
//
// A forward: route on the GPU over all E experts (handle `route`), read the
// selection back, copy in the experts that are not resident, rename the
// selection to arena slots and run the expert kernels over the arena (handle
// `arena`, whose "experts" are the slots). The kernels and their data are the
// ones k3moe_layer_forward uses, so the results are the same bit for bit.
//
// A device-planned cache keeps the residency tables in device memory
// instead: a one-workgroup kernel plans each call with the same rule, and a
// fill kernel copies the missing experts from pinned host memory over PCIe
// (cache_plan.hip). A forward is then only enqueued (no read-back), so it can
// run ahead of the GPU and be captured in a graph.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <new>
#include <vector>

#include "k3_kernels.h"
#include "k3moe.h"
#include "k3moe_internal.h"
#include "lru.h"

namespace {

constexpr int kTensors = k3::kCacheTensors;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bytes of one expert's share of each tiled tensor.
void expert_bytes(const k3moe_config* c, size_t (&b)[kTensors]) {
  const int32_t d = c->d_model, f = c->d_ff;
  b[0] = (size_t)f * d / 2;
  b[1] = (size_t)k3moe_tiled_scale_bytes(1, f, d);
  b[2] = b[0];
  b[3] = b[1];
  b[4] = (size_t)d * f / 2;
  b[5] = (size_t)k3moe_tiled_scale_bytes(1, d, f);
}

}  // namespace

struct k3moe_cache {
  k3moe_config cfg;
  int device;
  int32_t n_slots;
  k3moe* route;  // router over all E experts (its expert pointers are never read)
  k3moe* arena;  // expert kernels over the n_slots arena slots
  uint8_t* mem;  // arena: tensor t of slot s at dev[t] + s * bytes[t]
  uint8_t* dev[kTensors];
  const uint8_t* host[kTensors];
  size_t bytes[kTensors];
  size_t expert_total;
  int32_t* idx_dev;    // [max_tokens][k] expert ids from the router
  float* gate_dev;     // [max_tokens][k]
  int32_t* sidx_dev;   // [max_tokens][k] the same selection as slot ids
  int32_t* idx_host;   // pinned copies
  int32_t* sidx_host;
  k3::ExpertLru lru;               // which slot holds which expert, and the replacement rule
  std::vector<k3::SlotCopy> copies;  // scratch: the copies a call or prefetch plans
  hipEvent_t pf_ev;                // recorded after the last prefetch's copies
  bool pf_pending;                 // the next forward must wait for pf_ev
  int64_t calls, hits, misses, bytes_in;  // completed calls and their experts
  int64_t prefetched, pf_hits;     // experts copied by prefetches; hits on them
  // device-planned caches: the tables live on the device and the host keeps
  // only what orders the calls' kernels across streams
  bool device_plan;
  void* tab_mem;                   // the tables' allocation
  float* logits_dev;               // [max_tokens][E] router logits (device-planned)
  const float* sel_bias;           // the router bias when it only ranks the experts, else NULL
  k3::CacheTables tb;
  k3::FillPlan fp;
  hipEvent_t plan_ev;              // recorded after the last plan kernel
  hipStream_t plan_stream;         // its stream
  unsigned long long plan_cap;     // its stream's capture id (0: not capturing)
  bool plan_recorded;
  hipStream_t pf_stream;           // stream and capture id of pf_ev's record
  unsigned long long pf_cap;
};

namespace {

struct Guard {
  int prev = -1;
  bool ok = false;
  explicit Guard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) return;
    ok = (prev == dev) || (hipSetDevice(dev) == hipSuccess);
  }
  ~Guard() {
    if (ok && prev >= 0) (void)hipSetDevice(prev);
  }
};

void release(k3moe_cache* c) {
  if (c->pf_ev) (void)hipEventDestroy(c->pf_ev);
  if (c->plan_ev) (void)hipEventDestroy(c->plan_ev);
  (void)hipFree(c->tab_mem);
  (void)hipFree(c->logits_dev);
  k3moe_destroy(c->route);
  k3moe_destroy(c->arena);
  (void)hipFree(c->mem);
  (void)hipFree(c->idx_dev);
  (void)hipFree(c->gate_dev);
  (void)hipFree(c->sidx_dev);
  (void)hipHostFree(c->idx_host);
  (void)hipHostFree(c->sidx_host);
}

// Copy expert e into slot v on stream st (the six tensors); the caller
// updates the residency tables.
hipError_t copy_in(k3moe_cache* c, int32_t e, int32_t v, hipStream_t st) {
  for (int t = 0; t < kTensors; ++t) {
    const hipError_t r =
        hipMemcpyAsync(c->dev[t] + (size_t)v * c->bytes[t], c->host[t] + (size_t)e * c->bytes[t],
                       c->bytes[t], hipMemcpyHostToDevice, st);
    if (r != hipSuccess) return r;
  }
  return hipSuccess;
}

// Device tables: every slot empty, nothing used, counters kept unless
// `counters` (at create).
hipError_t reset_tables(k3moe_cache* c, bool counters) {
  const size_t E = (size_t)c->cfg.n_experts, S = (size_t)c->n_slots;
  hipError_t r = hipMemset(c->tb.slot_of, 0xff, E * 4);
  if (r == hipSuccess) r = hipMemset(c->tb.expert_in, 0xff, S * 4);
  if (r == hipSuccess) r = hipMemset(c->tb.last_use, 0, S * 8);
  if (r == hipSuccess) r = hipMemset(c->tb.pre, 0, S * 4);
  if (r == hipSuccess) r = hipMemset(c->tb.fwd_copies, 0, 4);
  if (r == hipSuccess) r = hipMemset(c->tb.pf_copies, 0, 4);
  if (r == hipSuccess && counters) r = hipMemset(c->tb.fwd_use, 0, S * 8);
  if (r == hipSuccess && counters) r = hipMemset(c->tb.ctr, 0, k3::kCacheCounters * 8);
  return r;
}

// A failed forward or prefetch: wait for whatever it enqueued on st (so no
// copy of it is still in flight when another stream reuses a slot), clear the
// error and forget every resident expert.
int fail(k3moe_cache* c, int rc, hipStream_t st) {
  (void)hipStreamSynchronize(st);
  (void)hipGetLastError();
  if (c->device_plan) {
    (void)hipDeviceSynchronize();
    (void)reset_tables(c, false);
    (void)hipGetLastError();
    c->plan_recorded = false;
    c->pf_pending = false;
  } else {
    c->lru.forget();
  }
  return rc;
}

// Capture id of st (0 when it is not capturing); false if it cannot be told.
bool capture_id(hipStream_t st, unsigned long long& id) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  id = 0;
  if (hipStreamGetCaptureInfo(st, &cs, &id) != hipSuccess) return false;
  if (cs != hipStreamCaptureStatusActive) id = 0;
  return true;
}

// Makes st wait for an event recorded on another stream, when that record is
// on the same timeline as st's work: both eager, or both in one capture. (An
// eager call does not wait on a record inside a graph, nor a captured call on
// an eager record: the caller orders graphs and eager calls.)
hipError_t wait_other(hipStream_t st, unsigned long long cap, hipEvent_t ev, hipStream_t ev_st,
                      unsigned long long ev_cap) {
  if (ev_st == st || ev_cap != cap) return hipSuccess;
  return hipStreamWaitEvent(st, ev, 0);
}

// Device-planned calls: the plan kernel runs after the previous plan kernel,
// whatever its stream; then the event marks this one.
hipError_t plan_begin(k3moe_cache* c, hipStream_t st, unsigned long long cap) {
  if (!c->plan_recorded) return hipSuccess;
  return wait_other(st, cap, c->plan_ev, c->plan_stream, c->plan_cap);
}
hipError_t plan_end(k3moe_cache* c, hipStream_t st, unsigned long long cap) {
  const hipError_t r = hipEventRecord(c->plan_ev, st);
  if (r != hipSuccess) return r;
  c->plan_stream = st;
  c->plan_cap = cap;
  c->plan_recorded = true;
  return hipSuccess;
}

// The device pointer of pinned host memory (0 if p is not pinned host memory).
const uint8_t* device_view(const uint8_t* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess || a.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, const_cast<uint8_t*>(p), 0) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return static_cast<const uint8_t*>(d);
}

// The device-planned forward (the checks of k3moe_cache_forward are done).
int forward_device_planned(k3moe_cache* c, const void* x, int32_t T, float* y, int32_t* topk_idx,
                           float* topk_gate, hipStream_t st) {
  const int P = T * c->cfg.top_k;
  const int E = c->cfg.n_experts, S = c->n_slots;
  unsigned long long cap = 0;
  if (!capture_id(st, cap)) return fail(c, K3MOE_EHIP, st);
  // 1. router logits over all experts (nothing read back)
  int rc = k3::route_logits(c->route, x, T, c->logits_dev, st);
  if (rc != K3MOE_OK) return fail(c, rc, st);
  // 2. an earlier prefetch's copies land, and the previous plan has run,
  // before this plan reads the tables; then the top k and the plan in one
  // kernel (which also writes the caller's idx and gate), and the copies of
  // the misses
  if (c->pf_pending && wait_other(st, cap, c->pf_ev, c->pf_stream, c->pf_cap) != hipSuccess)
    return fail(c, K3MOE_EHIP, st);
  c->pf_pending = false;
  if (plan_begin(c, st, cap) != hipSuccess ||
      k3::launch_cache_plan_forward(c->logits_dev, T, c->cfg.top_k, c->sel_bias, E, S, c->tb,
                                    c->idx_dev, c->gate_dev, topk_idx, topk_gate, c->sidx_dev,
                                    st) != hipSuccess ||
      plan_end(c, st, cap) != hipSuccess ||
      k3::launch_cache_fill(c->tb.fwd_copies, P, E, S, c->fp, st) != hipSuccess)
    return fail(c, K3MOE_EHIP, st);
  // 3. the expert kernels over the arena, with the selection renamed to slots
  rc = k3moe_experts_forward(c->arena, x, T, c->sidx_dev, c->gate_dev, y, st);
  if (rc != K3MOE_OK) return fail(c, rc, st);
  return K3MOE_OK;
}

}  // namespace

extern "C" {

int k3moe_cache_create(const k3moe_config* cfg, const k3moe_host_weights* w, int32_t n_slots,
                       int device, k3moe_cache** out) {
  return k3moe_cache_create_ex(cfg, w, n_slots, device, 0u, out);
}

int k3moe_cache_create_ex(const k3moe_config* cfg, const k3moe_host_weights* w, int32_t n_slots,
                          int device, uint32_t flags, k3moe_cache** out) {
  if (out) *out = nullptr;
  if (!out || !w || !cfg) return K3MOE_EINVAL;
  if (flags & ~(uint32_t)K3MOE_CACHE_DEVICE_PLAN) return K3MOE_EINVAL;
  const bool device_plan = (flags & K3MOE_CACHE_DEVICE_PLAN) != 0;
  const int64_t ws = k3moe_workspace_bytes(cfg);  // validates cfg on the host
  if (ws < 0) return (int)ws;
  if (n_slots < cfg->top_k || n_slots > cfg->n_experts) return K3MOE_EINVAL;
  if (!w->router_w || !aligned16(w->router_w)) return K3MOE_EINVAL;
  if (w->router_b && !aligned16(w->router_b)) return K3MOE_EINVAL;
  const uint8_t* hp[kTensors] = {w->gate_q, w->gate_s, w->up_q, w->up_s, w->down_q, w->down_s};
  for (const uint8_t* p : hp)
    if (!p) return K3MOE_EINVAL;
  if (device_plan)
    for (const uint8_t* p : hp)
      if (!aligned16(p)) return K3MOE_EINVAL;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) return K3MOE_EHIP;
  if (device < 0 || device >= ndev) return K3MOE_EINVAL;
  Guard guard(device);
  if (!guard.ok) return K3MOE_EHIP;
  // a device-planned cache reads the host tensors from its kernels: they must
  // be pinned host memory the device can address
  const uint8_t* hview[kTensors] = {};
  if (device_plan)
    for (int t = 0; t < kTensors; ++t)
      if (!(hview[t] = device_view(hp[t]))) return K3MOE_EINVAL;

  k3moe_cache* c = new (std::nothrow) k3moe_cache();
  if (!c) return K3MOE_ENOMEM;
  c->cfg = *cfg;
  c->device = device;
  c->n_slots = n_slots;
  c->device_plan = device_plan;
  expert_bytes(cfg, c->bytes);
  c->expert_total = 0;
  for (int t = 0; t < kTensors; ++t) {
    c->host[t] = hp[t];
    c->expert_total += c->bytes[t];  // each a multiple of 256 (1 KB code tiles, 256 B scale groups)
  }
  // arena: six tensors of n_slots experts, each tensor 256-byte aligned
  size_t off[kTensors], total = 0;
  for (int t = 0; t < kTensors; ++t) {
    off[t] = total;
    total += ((size_t)n_slots * c->bytes[t] + 255) / 256 * 256;
  }
  const size_t P = (size_t)cfg->max_tokens * cfg->top_k;
  size_t free_b = 0, total_b = 0;
  if (hipMemGetInfo(&free_b, &total_b) != hipSuccess) {
    delete c;
    return K3MOE_EHIP;
  }
  // device tables: slot_of [E], expert_in [S], last_use [S], fwd_use [S],
  // pre [S], counters, two copy lists of 1 + 2 S
  const size_t E = (size_t)cfg->n_experts, S = (size_t)n_slots;
  const size_t tab_bytes = device_plan ? E * 4 + S * 4 + S * 8 + S * 8 + S * 4 +
                                             k3::kCacheCounters * 8 + 2 * (1 + 2 * S) * 4 + 64
                                       : 0;
  const size_t logit_bytes = device_plan ? (size_t)cfg->max_tokens * E * 4 : 0;
  // refuse before allocating: the arena, two workspaces, the selection buffers
  if (total + 2 * (size_t)ws + 3 * P * 4 + tab_bytes + logit_bytes > free_b) {
    delete c;
    return K3MOE_ENOMEM;
  }
  void* m = nullptr;
  bool ok = hipMalloc(&m, total) == hipSuccess;
  c->mem = static_cast<uint8_t*>(m);
  ok = ok && hipMalloc(reinterpret_cast<void**>(&c->idx_dev), P * 4) == hipSuccess;
  ok = ok && hipMalloc(reinterpret_cast<void**>(&c->gate_dev), P * 4) == hipSuccess;
  ok = ok && hipMalloc(reinterpret_cast<void**>(&c->sidx_dev), P * 4) == hipSuccess;
  ok = ok && hipHostMalloc(reinterpret_cast<void**>(&c->idx_host), P * 4, 0) == hipSuccess;
  ok = ok && hipHostMalloc(reinterpret_cast<void**>(&c->sidx_host), P * 4, 0) == hipSuccess;
  if (ok && device_plan) {
    ok = hipMalloc(&c->tab_mem, tab_bytes) == hipSuccess &&
         hipMalloc(reinterpret_cast<void**>(&c->logits_dev), logit_bytes) == hipSuccess;
    if (ok) {
      // 8-byte fields first, then the 4-byte ones
      int64_t* p8 = static_cast<int64_t*>(c->tab_mem);
      c->tb.ctr = p8;
      c->tb.last_use = p8 + k3::kCacheCounters;
      c->tb.fwd_use = c->tb.last_use + S;
      int32_t* p4 = reinterpret_cast<int32_t*>(c->tb.fwd_use + S);
      c->tb.slot_of = p4;
      c->tb.expert_in = p4 + E;
      c->tb.pre = c->tb.expert_in + S;
      c->tb.fwd_copies = c->tb.pre + S;
      c->tb.pf_copies = c->tb.fwd_copies + 1 + 2 * S;
    }
  }
  if (!ok) {
    (void)hipGetLastError();
    release(c);
    delete c;
    return K3MOE_ENOMEM;
  }
  for (int t = 0; t < kTensors; ++t) c->dev[t] = c->mem + off[t];
  if (device_plan) {
    for (int t = 0; t < kTensors; ++t) {
      c->fp.src[t] = hview[t];
      c->fp.dst[t] = c->dev[t];
      c->fp.bytes[t] = c->bytes[t];
    }
    c->fp.total = c->expert_total;
    c->sel_bias = (cfg->flags & K3MOE_FLAG_BIAS_SELECT_ONLY) ? w->router_b : nullptr;
    if (reset_tables(c, true) != hipSuccess ||
        k3::prepare_cache_plan((int)std::min(P, S), (int)E, (int)S) != hipSuccess ||
        hipEventCreateWithFlags(&c->plan_ev, hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      release(c);
      delete c;
      return K3MOE_EHIP;
    }
  }
  // the router handle sees all E experts; the arena handle sees the slots
  k3moe_weights rw = {w->router_w, w->router_b, c->dev[0], c->dev[1], c->dev[2],
                      c->dev[3],   c->dev[4],   c->dev[5]};
  k3moe_config acfg = *cfg;
  acfg.n_experts = n_slots;
  int rc = k3moe_create(cfg, &rw, device, &c->route);
  if (rc == K3MOE_OK) rc = k3moe_create(&acfg, &rw, device, &c->arena);
  if (rc != K3MOE_OK) {
    release(c);
    delete c;
    return rc;
  }
  c->lru.reset(cfg->n_experts, n_slots);
  c->copies.reserve((size_t)n_slots);
  c->calls = c->hits = c->misses = c->bytes_in = 0;
  c->prefetched = c->pf_hits = 0;
  c->pf_pending = false;
  if (hipEventCreateWithFlags(&c->pf_ev, hipEventDisableTiming) != hipSuccess) {
    c->pf_ev = nullptr;
    (void)hipGetLastError();
    release(c);
    delete c;
    return K3MOE_EHIP;
  }
  *out = c;
  return K3MOE_OK;
}

void k3moe_cache_destroy(k3moe_cache* c) {
  if (!c) return;
  {
    Guard guard(c->device);
    if (guard.ok) {
      (void)hipDeviceSynchronize();
      release(c);
    }
  }
  delete c;
}

namespace {

// The device tables' counters, after everything enqueued on the device.
int read_counters(const k3moe_cache* c, int64_t (&v)[k3::kCacheCounters]) {
  Guard guard(c->device);
  if (!guard.ok) return K3MOE_EHIP;
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(v, c->tb.ctr, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) {
    (void)hipGetLastError();
    return K3MOE_EHIP;
  }
  return K3MOE_OK;
}

}  // namespace

int k3moe_cache_stats(const k3moe_cache* c, int64_t* calls, int64_t* hits, int64_t* misses,
                      int64_t* bytes_in) {
  if (!c) return K3MOE_EINVAL;
  if (c->device_plan) {
    int64_t v[k3::kCacheCounters];
    const int rc = read_counters(c, v);
    if (rc != K3MOE_OK) return rc;
    if (calls) *calls = v[k3::kCtrCalls];
    if (hits) *hits = v[k3::kCtrHits];
    if (misses) *misses = v[k3::kCtrMisses];
    if (bytes_in)
      *bytes_in = (v[k3::kCtrMisses] + v[k3::kCtrPrefetched]) * (int64_t)c->expert_total;
    return K3MOE_OK;
  }
  if (calls) *calls = c->calls;
  if (hits) *hits = c->hits;
  if (misses) *misses = c->misses;
  if (bytes_in) *bytes_in = c->bytes_in;
  return K3MOE_OK;
}

int k3moe_cache_prefetch_device(k3moe_cache* c, const int32_t* experts, int32_t n, void* stream) {
  if (!c || !c->device_plan || n < 0 || (n > 0 && !experts)) return K3MOE_EINVAL;
  if (n > 0 && (reinterpret_cast<uintptr_t>(experts) & 3u)) return K3MOE_EINVAL;
  if (n == 0) return K3MOE_OK;
  Guard guard(c->device);
  if (!guard.ok) return K3MOE_EHIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned long long cap = 0;
  if (!capture_id(st, cap)) return fail(c, K3MOE_EHIP, st);
  // the copies of a previous prefetch on another stream land first (a
  // forward after this one waits only for this prefetch's event)
  if (c->pf_pending && wait_other(st, cap, c->pf_ev, c->pf_stream, c->pf_cap) != hipSuccess)
    return fail(c, K3MOE_EHIP, st);
  const int E = c->cfg.n_experts, S = c->n_slots;
  if (plan_begin(c, st, cap) != hipSuccess ||
      k3::launch_cache_plan_prefetch(experts, n, E, S, c->tb, st) != hipSuccess ||
      plan_end(c, st, cap) != hipSuccess ||
      k3::launch_cache_fill(c->tb.pf_copies, S, E, S, c->fp, st) != hipSuccess ||
      hipEventRecord(c->pf_ev, st) != hipSuccess)
    return fail(c, K3MOE_EHIP, st);
  c->pf_pending = true;
  c->pf_stream = st;
  c->pf_cap = cap;
  return K3MOE_OK;
}

int k3moe_cache_device_counters(const k3moe_cache* c, int64_t* refused_prefetches,
                                int64_t* ignored_ids) {
  if (!c || !c->device_plan) return K3MOE_EINVAL;
  int64_t v[k3::kCacheCounters];
  const int rc = read_counters(c, v);
  if (rc != K3MOE_OK) return rc;
  if (refused_prefetches) *refused_prefetches = v[k3::kCtrPfRefused];
  if (ignored_ids) *ignored_ids = v[k3::kCtrIgnored];
  return K3MOE_OK;
}

int k3moe_cache_forward(k3moe_cache* c, const void* x, int32_t T, float* y, int32_t* topk_idx,
                        float* topk_gate, void* stream) {
  if (!c) return K3MOE_EINVAL;
  if (T < 0 || T > c->cfg.max_tokens) return K3MOE_EINVAL;
  if (T == 0) return K3MOE_OK;
  if (!x || !y || !aligned16(x) || !aligned16(y)) return K3MOE_EINVAL;
  if ((topk_idx && (reinterpret_cast<uintptr_t>(topk_idx) & 3u)) ||
      (topk_gate && (reinterpret_cast<uintptr_t>(topk_gate) & 3u)))
    return K3MOE_EINVAL;
  Guard guard(c->device);
  if (!guard.ok) return K3MOE_EHIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t P = (size_t)T * c->cfg.top_k;
  if (c->device_plan) {
    // every call fits in the arena: at most T*k distinct experts
    if (P > (size_t)c->n_slots) return K3MOE_EUNSUPPORTED;
    return forward_device_planned(c, x, T, y, topk_idx, topk_gate, st);
  }

  // 1. route over all experts and read the selection back
  int rc = k3moe_route(c->route, x, T, nullptr, c->idx_dev, c->gate_dev, stream);
  if (rc != K3MOE_OK) return fail(c, rc, st);
  if (hipMemcpyAsync(c->idx_host, c->idx_dev, P * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    (void)hipGetLastError();
    return fail(c, K3MOE_EHIP, st);
  }

  // 2. plan the call: its distinct experts, the hits, and for each miss the
  // least recently used slot the call does not use. Refused, with nothing
  // changed, if they cannot all be resident at once.
  int64_t hits = 0, misses = 0, pf_hits = 0;
  if (!c->lru.plan_forward(c->idx_host, P, c->copies, hits, misses, pf_hits))
    return K3MOE_EUNSUPPORTED;
  // copies of an earlier prefetch (possibly on another stream) land before
  // this call copies into, or reads, any slot
  if (c->pf_pending) {
    if (hipStreamWaitEvent(st, c->pf_ev, 0) != hipSuccess) {
      (void)hipGetLastError();
      return fail(c, K3MOE_EHIP, st);
    }
    c->pf_pending = false;
  }
  // 3. the misses' copies, on the call's stream
  for (const k3::SlotCopy& cp : c->copies)
    if (copy_in(c, cp.expert, cp.slot, st) != hipSuccess) {
      (void)hipGetLastError();
      return fail(c, K3MOE_EHIP, st);
    }
  // 4. the selection renamed to slots (dropped pairs stay out of range)
  c->lru.rename(c->idx_host, P, c->sidx_host);
  if (hipMemcpyAsync(c->sidx_dev, c->sidx_host, P * 4, hipMemcpyHostToDevice, st) != hipSuccess) {
    (void)hipGetLastError();
    return fail(c, K3MOE_EHIP, st);
  }
  // 5. the expert kernels over the arena
  rc = k3moe_experts_forward(c->arena, x, T, c->sidx_dev, c->gate_dev, y, stream);
  if (rc != K3MOE_OK) return fail(c, rc, st);
  if ((topk_idx && hipMemcpyAsync(topk_idx, c->idx_dev, P * 4, hipMemcpyDeviceToDevice, st) !=
                       hipSuccess) ||
      (topk_gate && hipMemcpyAsync(topk_gate, c->gate_dev, P * 4, hipMemcpyDeviceToDevice, st) !=
                        hipSuccess)) {
    (void)hipGetLastError();
    return fail(c, K3MOE_EHIP, st);
  }
  ++c->calls;
  c->hits += hits;
  c->misses += misses;
  c->pf_hits += pf_hits;
  c->bytes_in += misses * (int64_t)c->expert_total;
  return K3MOE_OK;
}

int k3moe_cache_prefetch(k3moe_cache* c, const int32_t* experts, int32_t n, void* stream) {
  if (!c || n < 0 || (n > 0 && !experts) || c->device_plan) return K3MOE_EINVAL;
  const int32_t E = c->cfg.n_experts;
  for (int32_t i = 0; i < n; ++i)
    if (experts[i] < 0 || experts[i] >= E) return K3MOE_EINVAL;
  if (n == 0) return K3MOE_OK;
  Guard guard(c->device);
  if (!guard.ok) return K3MOE_EHIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // slots a prefetch may fill: not used by the last forward (its kernels may
  // still run) and not taken by this prefetch; refused, with nothing
  // changed, if too few are left for the listed experts that are not
  // resident
  const k3::ExpertLru::PrefetchPlan plan = c->lru.plan_prefetch(experts, n, c->copies);
  if (plan == k3::ExpertLru::kRefused) return K3MOE_EUNSUPPORTED;
  if (plan == k3::ExpertLru::kBroken) {
    c->pf_pending = false;
    return fail(c, K3MOE_EUNSUPPORTED, st);
  }
  int64_t copied = 0;
  for (const k3::SlotCopy& cp : c->copies) {
    if (copy_in(c, cp.expert, cp.slot, st) != hipSuccess) {
      c->pf_pending = false;
      return fail(c, K3MOE_EHIP, st);
    }
    ++copied;
  }
  if (hipEventRecord(c->pf_ev, st) != hipSuccess) {
    (void)hipGetLastError();
    return fail(c, K3MOE_EHIP, st);
  }
  c->pf_pending = true;
  c->prefetched += copied;
  c->bytes_in += copied * (int64_t)c->expert_total;
  return K3MOE_OK;
}

int k3moe_cache_prefetch_stats(const k3moe_cache* c, int64_t* prefetched, int64_t* prefetch_hits) {
  if (!c) return K3MOE_EINVAL;
  if (c->device_plan) {
    int64_t v[k3::kCacheCounters];
    const int rc = read_counters(c, v);
    if (rc != K3MOE_OK) return rc;
    if (prefetched) *prefetched = v[k3::kCtrPrefetched];
    if (prefetch_hits) *prefetch_hits = v[k3::kCtrPfHits];
    return K3MOE_OK;
  }
  if (prefetched) *prefetched = c->prefetched;
  if (prefetch_hits) *prefetch_hits = c->pf_hits;
  return K3MOE_OK;
}

}  // extern "C"
