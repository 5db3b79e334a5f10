/*
 * k3moe.h - C ABI of the MI355X (gfx950) forward pass of one sparse
 * Mixture-of-Experts layer whose expert weights are stored in MXFP4.
 *
 * The layer is the MoE block of the Kimi K3 model that the kimi-k3-in-c pages
 * describe: a router picks the top 16 of 896 routed experts per token
 * (CHANGELOG walk-through, 0.1.0 section: "MoE router, top-16 of 896"), each
 * expert is a gated-linear (SwiGLU) FFN (same section, printed "SiTU-GLU"),
 * and expert weights are 4-bit E2M1 codes with a shared E8M0 scale per 32
 * elements, consumed as packed nibbles (same section: "MXFP4 matmul consumes
 * packed nibbles directly"; "four reductions" overview: experts are already
 * nibbles, about half a byte per parameter). Tokens routed to the same expert
 * are grouped so each expert's weights are read once per call (CHANGELOG
 * walk-through, Unreleased section: chunk-union prefill, identical output to
 * the per-token path).
 *
 * What one forward computes, per token t (x[t] is bf16, everything else fp32):
 *   l[e]   = sum_i x[t,i] * Wr[e,i]  (+ bias[e])                  router logits
 *   S      = the k experts with the largest l, ties to the lower index,
 *            ordered by (l descending, index ascending)
 *   gate_j = exp(l_j - l_max) / sum_{i in S} exp(l_i - l_max)     renormalised
 *   for j in S:  g = Wg_j x, u = Wu_j x, h = SiLU(g) * u,  o_j = Wd_j h
 *   y[t]   = sum_j gate_j * o_j
 * with SiLU(z) = z / (1 + e^-z). The pages leave the router function, tie
 * rule and normalisation open; the readings above are the plainest ones.
 *
 * Conventions shared by every entry point
 * - Pointers are DEVICE pointers on the handle's device unless marked HOST.
 * - Every argument is checked before anything is enqueued; a failed check
 *   returns K3MOE_EINVAL (or K3MOE_EUNSUPPORTED) and writes nothing. The
 *   library never aborts, exits or prints (the pages' engine rejects bad
 *   input loudly instead of defaulting: CHANGELOG walk-through, config
 *   reader that refuses unknown configs).
 * - Work is enqueued on the caller's HIP stream (NULL = the legacy default
 *   stream) in stream order, with no host synchronisation. Faults inside
 *   kernels surface at the caller's next synchronisation.
 * - A handle owns one workspace; calls on one handle must not overlap (use one
 *   handle per concurrent stream).
 * - T = 0 is valid and does nothing.
 * - NaN/Inf inputs are not checked and propagate, except in the router: a
 *   NaN logit counts as -inf. In the selection it ranks equal to -inf (ties
 *   to the lower index), so it is chosen only when fewer than k logits lie
 *   above -inf; in the gates a selected one gets gate 0. Selected indices
 *   therefore always lie in [0, E).
 * - An E8M0 scale byte 0xFF is NaN and propagates through the sums it
 *   enters: a NaN block in row m of an expert's down projection makes
 *   output m of the tokens routed to that expert NaN; one in its gate or up
 *   projection makes all outputs of those tokens NaN.
 */
#ifndef K3MOE_H
#define K3MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define K3MOE_OK             0
#define K3MOE_EINVAL        -1   /* bad argument: null pointer, bad size, misalignment */
#define K3MOE_ENOMEM        -2   /* device memory for the workspace is not available */
#define K3MOE_EHIP          -3   /* a HIP runtime call or kernel launch failed */
#define K3MOE_EUNSUPPORTED  -4   /* valid but outside what the library supports */

typedef struct k3moe k3moe;  /* opaque handle */

/* Layer shape (HOST struct, copied by k3moe_create).
 * Supported: d % 128 == 0 and 128 <= d <= 8192; f % 128 == 0 and
 * 128 <= f <= 4096; 1 <= k <= E <= 4096; k <= 64; 1 <= max_tokens,
 * max_tokens * k < 2^31, max_tokens * d <= 2^30 and max_tokens * k * f <= 2^30
 * (32-bit offsets into the prefill activation planes; at d=7168, k=16,
 * f=2048 that is up to 32768 tokens per call). Anything else returns
 * K3MOE_EINVAL (malformed: non-positive sizes, d or f not a multiple of 32,
 * k > E, unknown flags) or K3MOE_EUNSUPPORTED (well-formed but beyond
 * these limits). */
typedef struct {
  int32_t d_model;     /* d: hidden size */
  int32_t n_experts;   /* E: routed experts */
  int32_t top_k;       /* k: experts per token */
  int32_t d_ff;        /* f: expert FFN width */
  int32_t max_tokens;  /* largest T any later call may pass; sizes the workspace */
  uint32_t flags;      /* 0 or K3MOE_FLAG_BIAS_SELECT_ONLY; other bits are invalid */
} k3moe_config;

/* flags: where the router bias enters. By default (flags = 0) router_b is
 * added to every logit before both the selection and the gates (the plain
 * reading of "a per-expert router bias"). With K3MOE_FLAG_BIAS_SELECT_ONLY
 * it only ranks the experts: the top k are chosen by l[e] + bias[e] (fp32
 * add, same ties and NaN rule), and the gates are the softmax of the chosen
 * experts' unbiased l[e] about their largest (the alternative reading, as
 * aux-loss-free load-balancing biases are used). The pages give the skewed
 * workload's bias but not where it enters. k3moe_route's logits output is
 * then the unbiased l. Without a bias the two modes are the same. */
#define K3MOE_FLAG_BIAS_SELECT_ONLY 1u

/* Layer weights (HOST struct of DEVICE pointers). BORROWED: they must stay
 * valid and unchanged until k3moe_destroy; the library never writes or
 * frees them. Every pointer must be 16-byte aligned.
 *
 * MXFP4 (OCP Microscaling v1.0): E2M1 element codes with one E8M0 scale (byte
 * b means 2^(b-127), 0xFF is NaN) per 32 consecutive elements along K, the
 * reduction dimension; within a 32-element block, element 2i sits in the low
 * nibble of byte i. Expert matrices are stored in the TILED layout below
 * (k3moe_pack_mxfp4 builds it from the row-major layout codes [rows][K/2],
 * scales [rows][K/32]). For a matrix of R rows and K columns, RT = R/16,
 * KT = K/128, KG = ceil(KT/4):
 *   codes  : 16-row x 128-column tiles, tile (rt, kt) = 1024 bytes at offset
 *            (rt*KT + kt)*1024; in it, bytes [16*l, 16*l+16) with
 *            l = r + 16*g hold the block of row 16*rt + r, columns
 *            128*kt + 32*g .. +31;
 *   scales : groups of four K tiles, group (rt, kg) = 256 bytes at offset
 *            (rt*KG + kg)*256; in it, byte 4*l + j (l = r + 16*g) is the scale
 *            of the block of row 16*rt + r, columns 128*(4*kg+j) + 32*g .. +31
 *            (127 where 4*kg + j >= KT).
 * The E experts of one tensor are stacked: expert e's codes start at
 * e*R*K/2, its scales at e*RT*KG*256. One 1024-byte tile is one wave's
 * 16-byte-per-lane load and exactly one A operand of the gfx950 MX MFMA. */
typedef struct {
  const float*   router_w;  /* [E][d] fp32, row-major */
  const float*   router_b;  /* [E] fp32 added to every token's logits, or NULL */
  const uint8_t* gate_q;    /* gate projection codes, tiled, R = f, K = d */
  const uint8_t* gate_s;    /* gate projection scales, tiled */
  const uint8_t* up_q;      /* up projection codes, tiled, R = f, K = d */
  const uint8_t* up_s;      /* up projection scales, tiled */
  const uint8_t* down_q;    /* down projection codes, tiled, R = d, K = f */
  const uint8_t* down_s;    /* down projection scales, tiled */
} k3moe_weights;

/* Create a handle on HIP device `device`: validates cfg and w, checks free
 * device memory before allocating (refusing before allocating, as the pages'
 * engine does for an over-budget KV cache), allocates the workspace for
 * cfg->max_tokens tokens and derives the router weight split used by the
 * prefill router. On success *out receives the handle and K3MOE_OK is
 * returned; on any failure *out is set to NULL (when out is not NULL),
 * nothing stays allocated and an error code is returned. Synchronous. */
int k3moe_create(const k3moe_config* cfg, const k3moe_weights* w, int device,
                 k3moe** out);

/* Destroy a handle: synchronises the handle's device (so none of its kernels
 * is still running), frees the workspace and the handle. NULL-safe. Never
 * frees weights. */
void k3moe_destroy(k3moe* h);

/* Static text for a status code. Never NULL. */
const char* k3moe_status_str(int status);

/* Bytes of device workspace a handle with this config allocates, or a
 * negative status if cfg is invalid. HOST-only, no device call. */
int64_t k3moe_workspace_bytes(const k3moe_config* cfg);

/* The whole layer: router -> top-k -> grouping -> experts -> combine.
 *   x         [T][d] bf16 activations, 16-byte aligned
 *   T         0 <= T <= max_tokens
 *   y         [T][d] fp32 output, 16-byte aligned; fully overwritten
 *   topk_idx  [T][k] int32 selected experts in selection order, or NULL
 *   topk_gate [T][k] fp32 gates matching topk_idx, or NULL
 *   stream    hipStream_t, or NULL for the default stream
 * y must not alias x, the weights or the index/gate outputs. */
int k3moe_layer_forward(k3moe* h, const void* x, int32_t T, float* y,
                        int32_t* topk_idx, float* topk_gate, void* stream);

/* The whole layer for decode-sized calls, with no handle and no allocation:
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). It runs the
 * same kernels as k3moe_layer_forward does for T <= 4 (router, gate/up with
 * the top-k fused, down with the combine fused), on the CURRENT HIP device,
 * and keeps its scratch (router logits, SwiGLU output h, and the routing when
 * topk_idx/topk_gate are NULL) in a fixed 2 MiB device array that the library
 * holds on each device for the life of the process. It calls no allocating
 * routine. Every call on one device shares that array: calls that overlap on
 * one device (two streams, or two host threads) race and must be ordered by
 * the caller. The first call on a device takes the array's address and sets
 * the kernels' LDS limits there.
 *   cfg, w     as for k3moe_create (HOST structs; w holds DEVICE pointers on
 *              the current device); cfg->max_tokens bounds T as usual
 *   x, T, y    as for k3moe_layer_forward, 0 <= T <= 4
 *   topk_idx, topk_gate  [T][k] outputs, both given or both NULL
 * Returns K3MOE_EINVAL for malformed arguments, K3MOE_EUNSUPPORTED when T > 4
 * or the scratch needed, 256-byte aligned slices of T*E*4 bytes of logits,
 * T*k*f*4 of h and (routing not given) 2*T*k*4 of idx/gate, exceeds 2 MiB
 * (the K3 shape d=7168, E=896, k=16, f=2048 needs 0.54 MB at T = 4). */
int k3moe_layer_forward_noalloc(const k3moe_config* cfg, const k3moe_weights* w,
                                const void* x, int32_t T, float* y,
                                int32_t* topk_idx, float* topk_gate, void* stream);

/* Router step alone: fp32 logits, top-k selection with ties to the lower
 * index, and gates renormalised over the selection.
 *   logits [T][E] fp32 output, or NULL to skip writing them
 *   idx    [T][k] int32 output; gate [T][k] fp32 output (both required) */
int k3moe_route(k3moe* h, const void* x, int32_t T, float* logits,
                int32_t* idx, float* gate, void* stream);

/* Grouping step alone (the chunk-union step: each routed expert's tokens are
 * gathered so its weights are read once). Input idx [T][k] int32 with every
 * value in [0, E) and the k values of one token distinct (values outside
 * [0, E) are dropped: counted nowhere, absent from perm). With T == 0, idx
 * and perm may be NULL and counts/offsets are written as zeros. Outputs:
 *   counts  [E]    pairs routed to each expert
 *   offsets [E+1]  exclusive prefix sum of counts (offsets[E] = T*k)
 *   perm    [T*k]  pair ids p = t*k + j ordered by (expert, t, j)  */
int k3moe_group(k3moe* h, const int32_t* idx, int32_t T, int32_t* counts,
                int32_t* offsets, int32_t* perm, void* stream);

/* Expert step alone with the caller's routing: grouping, the expert FFNs and
 * the gate-weighted combine. idx/gate [T][k] as produced by k3moe_route
 * (same constraints as k3moe_group; any gate values are accepted). */
int k3moe_experts_forward(k3moe* h, const void* x, int32_t T,
                          const int32_t* idx, const float* gate, float* y,
                          void* stream);

/* Rearrange n stacked MXFP4 matrices from the row-major layout (codes
 * [n][R][K/2], scales [n][R][K/32]) into the tiled layout of k3moe_weights.
 * Requires R % 16 == 0, K % 128 == 0, n >= 1; tiled_codes needs n*R*K/2 bytes,
 * tiled_scales k3moe_tiled_scale_bytes(n, R, K) bytes; all four are DEVICE
 * pointers on the current HIP device, 16-byte aligned and non-overlapping.
 * Enqueued on `stream`; returns K3MOE_EINVAL for bad arguments. */
int k3moe_pack_mxfp4(const uint8_t* codes, const uint8_t* scales, int32_t n, int32_t R, int32_t K,
                     uint8_t* tiled_codes, uint8_t* tiled_scales, void* stream);

/* The same rearrangement from row-major matrices in HOST memory (codes
 * [n][R][K/2], scales [n][R][K/32], pinned or pageable) into the tiled
 * DEVICE tensors tiled_codes / tiled_scales (16-byte aligned, sizes as for
 * k3moe_pack_mxfp4), on the current HIP device: the way to load a
 * checkpoint's experts. The matrices cross PCIe a chunk at a time through a
 * device staging buffer of at most 32 MiB (at least one matrix), so loading
 * needs the tiled tensors plus that buffer, never a second full copy.
 * Enqueued on `stream`, then synchronised with it: returns once the tiled
 * tensors are written and the staging buffer is freed. K3MOE_EINVAL for bad
 * arguments, K3MOE_ENOMEM if the staging buffer cannot be allocated,
 * K3MOE_EHIP if a copy or launch fails (the tiled tensors are then
 * incomplete). */
int k3moe_pack_mxfp4_from_host(const uint8_t* codes, const uint8_t* scales, int32_t n, int32_t R,
                               int32_t K, uint8_t* tiled_codes, uint8_t* tiled_scales,
                               void* stream);

/* Bytes of tiled scales for n matrices of R x K (0 if the shape is invalid). */
int64_t k3moe_tiled_scale_bytes(int32_t n, int32_t R, int32_t K);

/* ---------------------------------------------------------------- expert cache
 * For models whose experts do not all fit in HBM. The pages' engine streams
 * the experts of its 2.78T-parameter model from NVMe through an LRU expert
 * cache in RAM, and counts as "true resident" only the hits on experts that
 * stayed in the cache from the previous step; raw hits also count experts
 * its prefetcher has just read in (ssnai.com decision guide; pomoai.com
 * architecture overview; xugj520.cn run notes, cache statistics;
 * chenxutan.com, the third reduction). Here the layer's expert weights stay
 * on the HOST and an HBM arena holds n_slots of them, replaced
 * least-recently-used. Each forward routes on the GPU, reads
 * the selection back to the host, copies the experts it misses into free or
 * least-recently-used slots (over PCIe, on the call's stream), and runs the
 * expert kernels on the arena with the selection renamed to slots. Results
 * equal k3moe_layer_forward on the same weights bit for bit (the same
 * kernels on the same data; only the place of the weights differs).
 * k3moe_cache_prefetch copies experts in ahead of the call that needs them
 * (the pages' prefetcher, for instance on a copy stream while the previous
 * call computes). A hit on such an expert is a raw hit but not a true
 * resident one, so the two rates differ by the prefetch hits. */
typedef struct k3moe_cache k3moe_cache;

/* Host-resident expert weights of a cached layer (HOST struct).
 *   router_w, router_b: DEVICE pointers as in k3moe_weights, router_b may be
 *     NULL; BORROWED until k3moe_cache_destroy.
 *   gate_q .. down_s: HOST pointers to the tiled layout of k3moe_weights
 *     ([E] experts, each contiguous), BORROWED until k3moe_cache_destroy and
 *     never written. Page-locked (pinned) memory lets the copies run at full
 *     PCIe rate; pageable memory works, slower. */
typedef struct {
  const float* router_w;
  const float* router_b;
  const uint8_t* gate_q;
  const uint8_t* gate_s;
  const uint8_t* up_q;
  const uint8_t* up_s;
  const uint8_t* down_q;
  const uint8_t* down_s;
} k3moe_host_weights;

/* Create a cached layer: cfg as for k3moe_create; n_slots experts in the HBM
 * arena, cfg->top_k <= n_slots <= cfg->n_experts. A call may route to at most
 * n_slots distinct experts (else K3MOE_EUNSUPPORTED, nothing run). Allocates
 * the arena (n_slots x the bytes of one expert) and two handles' workspaces;
 * K3MOE_ENOMEM if they do not fit. */
int k3moe_cache_create(const k3moe_config* cfg, const k3moe_host_weights* w, int32_t n_slots,
                       int device, k3moe_cache** out);

/* Forward of the cached layer; arguments as k3moe_layer_forward. The call
 * waits on the host for the routing (one device-to-host copy of T*k indices)
 * before it enqueues the expert copies and kernels, so it returns once those
 * are enqueued, not when they finish. Calls on one cache must use one stream
 * (or be ordered by the caller). A failed call waits for what it had
 * enqueued on its stream, then forgets every resident expert (the next call
 * copies what it needs again). */
int k3moe_cache_forward(k3moe_cache* c, const void* x, int32_t T, float* y, int32_t* topk_idx,
                        float* topk_gate, void* stream);

/* Counters since create (HOST outputs, any may be NULL): completed calls,
 * distinct experts found resident (hits, raw: prefetched ones included) and
 * copied in (misses) per call, and bytes copied by calls and prefetches. A
 * refused call counts nowhere. */
int k3moe_cache_stats(const k3moe_cache* c, int64_t* calls, int64_t* hits, int64_t* misses,
                      int64_t* bytes_in);

/* Prefetch: copy the listed experts (HOST array of n expert ids, repeats
 * allowed; n = 0 does nothing) that are not resident into the arena, on
 * `stream` (hipStream_t, NULL = default stream), and refresh the resident
 * ones in the LRU order. The copies go into the least recently used slots
 * that the last forward does not use (its kernels may still run), so a
 * prefetch may be issued on another stream while that forward computes. The
 * next k3moe_cache_forward waits for the copies before it copies into or
 * reads any slot. Prefetches must use one stream (or be ordered by the
 * caller). Errors: K3MOE_EINVAL for a NULL cache, n < 0 or an id outside
 * [0, E); K3MOE_EUNSUPPORTED, with nothing changed, if more experts need a
 * slot than such slots exist; K3MOE_EHIP if a copy cannot be enqueued (the
 * call then waits for the copies it had enqueued and the cache forgets every
 * resident expert). */
int k3moe_cache_prefetch(k3moe_cache* c, const int32_t* experts, int32_t n, void* stream);

/* Prefetch counters (HOST outputs, any may be NULL): experts copied in by
 * prefetches, and hits of completed calls on experts a prefetch brought in
 * and no call had used before. True resident hits = hits - prefetch_hits. */
int k3moe_cache_prefetch_stats(const k3moe_cache* c, int64_t* prefetched, int64_t* prefetch_hits);

/* Destroy: synchronises the device, frees the arena and both handles.
 * NULL-safe; never frees the weights. */
void k3moe_cache_destroy(k3moe_cache* c);

/* Device-planned cache: k3moe_cache_create_ex with flags =
 * K3MOE_CACHE_DEVICE_PLAN keeps the residency tables in device memory. A
 * forward then routes, plans (one workgroup, the same replacement rule and
 * counts as above, call for call), copies the missing experts from the host
 * tensors with a kernel that reads them over PCIe, and runs the expert
 * kernels, all enqueued on the call's stream with nothing read back: the call
 * returns at once, the host never waits, and forwards and device prefetches
 * can be captured into a HIP graph and replayed (each replay plans anew
 * against the tables as they then are). The tables and the arena are the
 * same ones a replay and an eager call use, so graphs and eager calls on one
 * cache must be ordered by the caller.
 *   Requirements: the six host tensors are pinned host memory (allocated with
 *   hipHostMalloc, or torch pin_memory), 16-byte aligned; else K3MOE_EINVAL.
 *   A forward must have T * top_k <= n_slots (so its distinct experts always
 *   fit), else K3MOE_EUNSUPPORTED before anything is enqueued.
 *   k3moe_cache_prefetch (host list) is K3MOE_EINVAL on such a cache; use
 *   k3moe_cache_prefetch_device. k3moe_cache_stats and
 *   k3moe_cache_prefetch_stats synchronise the device and read the device
 *   counters (bytes_in = (misses + prefetched) * one expert's bytes).
 *   flags = 0 gives the host-planned cache of k3moe_cache_create. */
#define K3MOE_CACHE_DEVICE_PLAN 1u
int k3moe_cache_create_ex(const k3moe_config* cfg, const k3moe_host_weights* w, int32_t n_slots,
                          int device, uint32_t flags, k3moe_cache** out);

/* Prefetch on a device-planned cache: experts is a DEVICE array of n int32
 * expert ids (for instance the routing of the next call, computed on the
 * device), read when the plan kernel runs; ids outside [0, E) are skipped and
 * counted. The same slot rule as k3moe_cache_prefetch; when too few slots
 * are eligible the prefetch is refused on the device (counted, nothing
 * changed). The next forward waits for its copies. Errors: K3MOE_EINVAL for a
 * NULL or host-planned cache, n < 0, or a NULL or misaligned list with n > 0;
 * K3MOE_EHIP if a launch fails (the cache then forgets every resident
 * expert). */
int k3moe_cache_prefetch_device(k3moe_cache* c, const int32_t* experts, int32_t n, void* stream);

/* Counters only a device-planned cache has (HOST outputs, any may be NULL):
 * prefetches refused for want of eligible slots, and prefetch ids skipped
 * for lying outside [0, E). Synchronises the device. K3MOE_EINVAL for a NULL
 * or host-planned cache. */
int k3moe_cache_device_counters(const k3moe_cache* c, int64_t* refused_prefetches,
                                int64_t* ignored_ids);

/* Stage timing, a profiling aid. Between k3moe_profile_begin and
 * k3moe_profile_end every forward records a HIP event before and after each
 * stage's kernel launch(es) on the call's own stream, for at most max_calls
 * launches per stage (later launches run untimed). k3moe_profile_end waits
 * for the recorded events and writes, per stage, the summed milliseconds and
 * the number of timed launches into HOST arrays of K3MOE_NUM_STAGES entries,
 * then releases the events. The stages: */
#define K3MOE_STAGE_ROUTER_LOGITS 0  /* router logits (one kernel) */
#define K3MOE_STAGE_TOPK          1  /* top-k + gates (one kernel) */
#define K3MOE_STAGE_GROUP         2  /* histogram, block prefix, expert scan, permute (four kernels) */
#define K3MOE_STAGE_QUANT_X       3  /* activation split for the MFMA path (one kernel) */
#define K3MOE_STAGE_GATEUP        4  /* gate/up projection + SwiGLU (one kernel) */
#define K3MOE_STAGE_COMBINE       5  /* gate-weighted sum of the k expert outputs (one kernel) */
#define K3MOE_STAGE_DOWN          6  /* down projection (one kernel; decode: fused with the combine) */
#define K3MOE_NUM_STAGES          7
int k3moe_profile_begin(k3moe* h, int32_t max_calls);
int k3moe_profile_end(k3moe* h, float* total_ms, int32_t* launches);
/* The same for the stages in stage_mask only (bit i: stage i; the others
 * record no events and report 0 launches). Each event pair sits between two
 * kernels on the stream and adds a few microseconds to the call, so timing
 * one kernel inside a timed loop disturbs that loop less than timing all
 * seven stages. k3moe_profile_begin(h, n) is stage_mask = all stages.
 * K3MOE_EINVAL for a NULL handle, max_calls outside [1, 2^20], or a mask
 * that is 0 or has bits at K3MOE_NUM_STAGES or above. */
int k3moe_profile_begin_stages(k3moe* h, int32_t max_calls, uint32_t stage_mask);

#ifdef __cplusplus
}
#endif

#endif /* K3MOE_H */
