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
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <new>
#include <vector>

#include "k3moe.h"
#include "lru.h"

namespace {

constexpr int kTensors = 6;  // gate codes, gate scales, up codes, up scales, down codes, down scales

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

// A failed forward or prefetch: wait for whatever it enqueued on st (so no
// copy of it is still in flight when another stream reuses a slot), clear the
// error and forget every resident expert.
int fail(k3moe_cache* c, int rc, hipStream_t st) {
  (void)hipStreamSynchronize(st);
  (void)hipGetLastError();
  c->lru.forget();
  return rc;
}

}  // namespace

extern "C" {

int k3moe_cache_create(const k3moe_config* cfg, const k3moe_host_weights* w, int32_t n_slots,
                       int device, k3moe_cache** out) {
  if (out) *out = nullptr;
  if (!out || !w || !cfg) return K3MOE_EINVAL;
  const int64_t ws = k3moe_workspace_bytes(cfg);  // validates cfg on the host
  if (ws < 0) return (int)ws;
  if (n_slots < cfg->top_k || n_slots > cfg->n_experts) return K3MOE_EINVAL;
  if (!w->router_w || !aligned16(w->router_w)) return K3MOE_EINVAL;
  if (w->router_b && !aligned16(w->router_b)) return K3MOE_EINVAL;
  const uint8_t* hp[kTensors] = {w->gate_q, w->gate_s, w->up_q, w->up_s, w->down_q, w->down_s};
  for (const uint8_t* p : hp)
    if (!p) return K3MOE_EINVAL;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) return K3MOE_EHIP;
  if (device < 0 || device >= ndev) return K3MOE_EINVAL;
  Guard guard(device);
  if (!guard.ok) return K3MOE_EHIP;

  k3moe_cache* c = new (std::nothrow) k3moe_cache();
  if (!c) return K3MOE_ENOMEM;
  c->cfg = *cfg;
  c->device = device;
  c->n_slots = n_slots;
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
  // refuse before allocating: the arena, two workspaces, the selection buffers
  if (total + 2 * (size_t)ws + 3 * P * 4 > free_b) {
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
  if (!ok) {
    (void)hipGetLastError();
    release(c);
    delete c;
    return K3MOE_ENOMEM;
  }
  for (int t = 0; t < kTensors; ++t) c->dev[t] = c->mem + off[t];
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

int k3moe_cache_stats(const k3moe_cache* c, int64_t* calls, int64_t* hits, int64_t* misses,
                      int64_t* bytes_in) {
  if (!c) return K3MOE_EINVAL;
  if (calls) *calls = c->calls;
  if (hits) *hits = c->hits;
  if (misses) *misses = c->misses;
  if (bytes_in) *bytes_in = c->bytes_in;
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
  if (!c || n < 0 || (n > 0 && !experts)) return K3MOE_EINVAL;
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
  if (prefetched) *prefetched = c->prefetched;
  if (prefetch_hits) *prefetch_hits = c->pf_hits;
  return K3MOE_OK;
}

}  // extern "C"
