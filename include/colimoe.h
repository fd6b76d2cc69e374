/*
 * colimoe.h - C ABI of the MI355X (gfx950) int4 routed-expert MoE layer.
 *
 * The layer (sources cited by page title and section):
 *   [A] "Colibrì: running a 744B MoE model on a laptop with 2400 lines of pure C"
 *       (kechuai.cn article)
 *   [P] "colibrì" project profile (gh.puless.com)
 *   [D] "colibrì: 1300 lines of C, a 25 GB laptop, a 744-billion-parameter model"
 *       (SSP GitHub Daily #091, jsqmd.com)
 *
 *   - a router picks k of E experts per token, 8 of 256 at the pages' scale
 *     ([A] §1 background; [D] §3);
 *   - each routed expert is an int4 container with one scale per 64 weights
 *     ([P] "aggressive optimisation, conservative correctness"), its three
 *     matrices stored side by side ([A] §2 technical mechanism);
 *   - at batch 1 the weights are dequantised and multiplied in floating point
 *     ([D] §4, highlight 4);
 *   - a shared expert runs for every token ([D] §3);
 *   - batched positions read each unique expert once ([A] §2, batch-union);
 *   - precision and routing never change silently ([A] §4): every call
 *     validates its arguments and returns a status; there is no fallback.
 *
 * Computed per token t with activations x[t] (fp32, length d):
 *   l[e]  = sum_c R[e][c] x[c] + b[e]                       (fp32 logits)
 *   idx   = the k largest l[e], larger first, exact ties to the lower e
 *   w_j   = exp(l[idx_j] - l[idx_0]) / sum_i exp(l[idx_i] - l[idx_0])
 *   y_e   = Wd_e (SiLU(Wg_e x) * (Wu_e x)),  W[r][c] = q[r][c] * s[r][c/64]
 *   r[t] += sum_j w_j y_{idx_j}  (ascending expert id)  + y_shared
 *
 * Conventions
 *   - Status: 0 = COLIMOE_OK, negative = error (colimoe_status_str()).
 *     Arguments are checked on the host before anything is enqueued; a
 *     rejected call has no effect.  A fault inside a kernel surfaces as
 *     COLIMOE_E_HIP at the next call that synchronises.
 *   - Ownership: the caller owns every device buffer (layer weights,
 *     workspace, inputs, outputs).  The library owns only its host context.
 *   - route/forward/rmsnorm enqueue on the context's HIP stream, allocate
 *     nothing and do not synchronise the host; the one exception is a
 *     forward on a layer loaded with colimoe_load_experts_host, which reads
 *     the call's routing on the host to fill the HBM expert cache.
 *   - A context is not thread-safe: use one per stream.
 *   - Device pointers must be 16-byte aligned, layer buffers 256-byte aligned.
 *   - A call with T == 0 does nothing and may pass NULL data pointers.
 */
#ifndef COLIMOE_H
#define COLIMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define COLIMOE_API __attribute__((visibility("default")))

enum colimoe_status {
  COLIMOE_OK = 0,
  COLIMOE_E_ARG = -1,        /* null / misaligned pointer, bad flag or index */
  COLIMOE_E_SHAPE = -2,      /* invalid shape, or T outside [0, max_tokens] */
  COLIMOE_E_NOT_LOADED = -3, /* layer has no weights loaded */
  COLIMOE_E_WORKSPACE = -4,  /* workspace missing or too small */
  COLIMOE_E_HIP = -5,        /* a HIP runtime call failed */
  COLIMOE_E_STATE = -6,      /* call out of order (e.g. load before create) */
};

/* Forward path selection. */
enum colimoe_forward_flags {
  COLIMOE_FWD_AUTO = 0,      /* BF16_MFMA for prefill-shaped calls (T*k >= 64*E,
                                on average 64 tokens per expert); otherwise FXP
                                when d >= 2048 and f >= 2048, else FP32 */
  COLIMOE_FWD_FP32 = 1,      /* int4 weights dequantised to fp32, fp32 FMA, fp32
                                accumulation ([D] §4, highlight 4) */
  COLIMOE_FWD_BF16_MFMA = 2, /* grouped GEMM on the matrix cores for many tokens
                                per expert ([D] §4, highlight 4: the int4 kernel
                                pays off on batches): tokens grouped by expert
                                through the union lists; weights dequantised to
                                bf16 as bf16(q*s), x and SiLU(g)*u rounded to
                                bf16 (round to nearest even), fp32 accumulation;
                                down outputs combined in fp32.  Any shape */
  COLIMOE_FWD_FXP = 3,       /* fixed-point activations: every 16 activations are
                                encoded as 23-bit integers with one power-of-two
                                scale (error <= 2^-22 of the group's largest
                                magnitude) and multiplied with the int4 weights
                                exactly by integer dot products; per 16 columns
                                the exact sum is rounded once to fp32, scaled by
                                the fp16 weight scale and accumulated in fp32.
                                Needs d >= 2048 and f >= 2048 (else E_SHAPE) */
};

/* Context options (colimoe_config.flags). */
enum colimoe_config_flags {
  COLIMOE_CFG_INT8 = 1, /* experts stored as int8 with one fp16 scale per 64
                           weights ([P] lessons on record and [D] §4 highlight 2:
                           the pages keep their MTP head in int8 because int4
                           lost too much precision there): the canonical blob
                           layout with one two's-complement byte per weight
                           (colimoe_expert_bytes() = 3*d*f*(1 + 2/64)).
                           Forward calls take any T on the fp32 path (AUTO or
                           FP32: dequantisation to fp32, fp32 accumulation;
                           each unique expert read once per call, a token's
                           bits independent of the others); the fixed-point
                           and bf16 paths return E_SHAPE */
};

typedef struct colimoe_config {
  int32_t d;          /* hidden size, multiple of 64 */
  int32_t f;          /* expert intermediate size, multiple of 64 */
  int32_t n_experts;  /* E, 1..1024 */
  int32_t top_k;      /* k, 1..min(E, 16) */
  int32_t n_layers;   /* layers the context can hold, >= 1 */
  int32_t n_shared;   /* always-on shared experts: 0 or 1 */
  int32_t group_size; /* must be 64 */
  int32_t max_tokens; /* largest T of any call, 1..65536 */
  uint32_t flags;     /* colimoe_config_flags: 0, or COLIMOE_CFG_INT8 */
} colimoe_config;

/* One layer's weights in host memory, canonical format.
 * A canonical expert blob (colimoe_expert_bytes() bytes) is
 *   [gate q: f*d/2 B][gate s: f*(d/64) fp16][up q: f*d/2 B][up s: f*(d/64) fp16]
 *   [down q: d*f/2 B][down s: d*(f/64) fp16]
 * with gate/up row-major [f][d] and down row-major [d][f] (rows = outputs);
 * byte i of a row holds element 2i in bits 0-3 and element 2i+1 in bits 4-7,
 * each a two's-complement int4; scale g of a row covers elements 64g..64g+63. */
typedef struct colimoe_layer_src {
  const float *router;    /* [E][d] fp32, required */
  const float *bias;      /* [E] fp32 additive logit bias, or NULL (= 0) */
  const uint8_t *experts; /* E canonical blobs back to back, required */
  const uint8_t *shared;  /* one canonical blob; required iff n_shared == 1 */
} colimoe_layer_src;

/* Batch-union lists (device int32 arrays), for a call with T tokens:
 *   n_unique[1]                 number of distinct experts U
 *   ids[min(E, T*k)]            the distinct experts, ascending
 *   offsets[min(E, T*k) + 1]    pairs of ids[u] are offsets[u] .. offsets[u+1]-1
 *   pair_token[T*k], pair_slot[T*k]  the (token, slot j) of each pair, ordered
 *                               by (expert, token)
 *   pair_of[T*k]                position of pair (t, j) at index t*k + j */
typedef struct colimoe_union {
  int32_t *n_unique;
  int32_t *ids;
  int32_t *offsets;
  int32_t *pair_token;
  int32_t *pair_slot;
  int32_t *pair_of;
} colimoe_union;

typedef struct colimoe_ctx colimoe_ctx;

/* Validate cfg and create a context bound to a HIP stream (NULL = default
 * stream).  Selects the current HIP device.  Errors: E_ARG, E_SHAPE, E_HIP. */
COLIMOE_API int colimoe_create(const colimoe_config *cfg, void *hip_stream, colimoe_ctx **out);

/* Free the host context.  Device buffers stay the caller's. */
COLIMOE_API void colimoe_destroy(colimoe_ctx *ctx);

/* Change the stream later calls enqueue on. */
COLIMOE_API int colimoe_set_stream(colimoe_ctx *ctx, void *hip_stream);

/* Sizes, for the caller to allocate.  Return 0 for an invalid cfg.
 *   expert_bytes    bytes of one expert blob (same canonical and on device)
 *   layer_bytes     device bytes one loaded layer needs (router, bias, experts)
 *   workspace_bytes device scratch route/forward need at max_tokens */
COLIMOE_API size_t colimoe_expert_bytes(const colimoe_config *cfg);
COLIMOE_API size_t colimoe_layer_bytes(const colimoe_config *cfg);
COLIMOE_API size_t colimoe_workspace_bytes(const colimoe_config *cfg);

/* Hand the context a caller-owned device workspace of >= workspace_bytes.
 * Errors: E_ARG (null/misaligned), E_WORKSPACE (too small). */
COLIMOE_API int colimoe_set_workspace(colimoe_ctx *ctx, void *dev, size_t bytes);

/* Load one layer ([A] §2: an expert's three matrices are adjacent and read
 * as one unit): copies router, bias and the E (+ shared) canonical blobs
 * from host memory into the caller-owned device buffer dev_dst (>=
 * layer_bytes, 256-byte aligned), repacked into the kernels' layout, and
 * records them for `layer`.  Synchronous: host buffers may be reused on
 * return.  Errors: E_ARG, E_SHAPE (layer out of range), E_HIP. */
COLIMOE_API int colimoe_load_experts(colimoe_ctx *ctx, int32_t layer, const colimoe_layer_src *src, void *dev_dst,
                         size_t dev_bytes);

/* Tiered placement for models whose experts do not all fit in HBM ([A] §2:
 * parameters are data moved between tiers by how often routing asks for them,
 * with a per-layer LRU cache, a learned hot set saved between runs, and the
 * next layer's router run one layer ahead; [D] §3: the routed experts stay on
 * disk and are read on demand into an LRU cache; [D] key tuning parameters:
 * --repin N re-places the hot experts every N tokens.  Here host RAM over
 * PCIe plays the disk and HBM the RAM).
 *
 * colimoe_expert_cache_bytes: device bytes of an expert cache of n_slots
 * slots (slot maps of every layer, a prediction scratch, then the slots); 0
 * for a bad config or n_slots < 1.  colimoe_host_layer_bytes: device bytes of
 * a host-resident layer (router and bias only).
 *
 * colimoe_set_expert_cache: the caller-owned device buffer (256-byte aligned)
 * the cache lives in, before any host-resident layer is loaded (E_STATE once
 * one is).  The slots are split evenly among the context's n_layers layers:
 * layer l owns slots_per_layer = n_slots / n_layers of them, with its own
 * least-recently-used order, so a layer's calls never evict another layer's
 * experts (a partition of a layer resident in HBM stays unused).  Resets all
 * counters and usage histograms.  Creates the two streams (default priority)
 * and the events the prefetch uses.  Errors: E_ARG, E_STATE, E_WORKSPACE
 * (room for less than one slot), E_HIP.
 *
 * colimoe_load_experts_host: as colimoe_load_experts, but the routed experts
 * are repacked into pinned host memory owned by the context (freed by
 * colimoe_destroy or when the layer is loaded again); router and bias go to
 * dev_dst (colimoe_host_layer_bytes); the shared expert takes the first slot
 * of the layer's partition for the layer's lifetime.  A forward on such a
 * layer first copies the routing to the host (this synchronises the stream),
 * adds the routing to the layer's usage histogram (tokens routed to each
 * expert), brings each missing expert into the least recently used
 * evictable slot of the layer's partition that the call does not need, and
 * then runs the same kernels, reading every expert from the cache: results
 * are bit-identical to the layer loaded with colimoe_load_experts.  A call
 * whose routing needs more evictable slots than the partition has returns
 * E_WORKSPACE.  colimoe_debug_expert on such a layer returns E_STATE.
 * Errors: E_ARG, E_SHAPE, E_STATE (no cache), E_WORKSPACE (slots_per_layer <
 * n_shared + top_k: no room for one token's experts), E_HIP.
 *
 * colimoe_cache_set_prefetch: one-layer-ahead prediction ([A] §2).  With
 * depth > 0, a forward call of up to 16 tokens on host-resident layer l whose
 * next layer l + 1 is host-resident also runs layer l + 1's router and top-k
 * on the call's input x (the router "one layer ahead"), on the cache's side
 * stream while layer l's kernels run; the host waits for that prediction
 * only, then starts copying, over PCIe on the cache's copy stream, the first
 * `depth` experts of each token's predicted top-k (its largest predicted
 * logits) that are absent from layer l + 1's partition.  A later call reading
 * or evicting such a slot waits for its copy only.  depth = 0 (the default)
 * turns prediction off; 1 <= depth <= top_k.  Prediction changes which experts
 * are in the cache, never the results.  Errors: E_ARG (depth out of range),
 * E_STATE (no cache).
 *
 * colimoe_cache_repin: learned pinning ([A] §2: the engine records which
 * experts the workload routes to and pins the hottest).  For every
 * host-resident layer, pins the n experts of its usage histogram with the
 * most tokens (ties to the lower id) in its partition, loading the absent
 * ones, and unpins the rest; pinned experts are never evicted.  Synchronises
 * the stream.  Errors: E_ARG, E_STATE (no cache), E_WORKSPACE (n > slots_per_layer
 * - n_shared - top_k: one token's experts must still fit), E_HIP.
 *
 * colimoe_cache_set_autorepin: repins a layer by itself ([D] key tuning
 * parameters, --repin N): every every_tokens tokens a host-resident layer has
 * served, its forward call first repins it with n (capped at slots_per_layer
 * - n_shared - top_k).  every_tokens = 0 turns it off (the default).
 * Errors: E_ARG, E_STATE (no cache), E_WORKSPACE (n too large).
 *
 * colimoe_cache_usage: the usage histogram of one layer (E counts: tokens
 * routed to each expert since the cache was set or the histogram loaded).
 * colimoe_cache_usage_save / _load: the histograms of all layers to / from a
 * file (the learned hot set kept between runs): 8 bytes "COLIUSE1", int32
 * n_layers, int32 E, then n_layers * E uint32 counts, little-endian.  Load
 * replaces the counts (a repin then pins by them).  Errors: E_ARG (null,
 * unreadable or unwritable file, not a usage file, truncated), E_SHAPE (the
 * file's layers or experts differ), E_STATE (no cache).
 *
 * colimoe_cache_stats: experts found in the cache and brought in on demand
 * since the cache was set, and its number of slots.  colimoe_cache_get_info:
 * those and the prediction figures: predicted = routed experts of calls that
 * had a prediction, predicted_hits = how many of them its full top-k named
 * (their ratio is the prediction hit rate); prefetched = experts copied ahead, and
 * prefetched_used = how many of those a call then needed; slots,
 * slots_per_layer, pinned (slots holding pinned experts).  Errors: E_ARG. */
typedef struct colimoe_cache_info {
  int64_t hits, misses;
  int64_t predicted, predicted_hits;
  int64_t prefetched, prefetched_used;
  int32_t slots, slots_per_layer, pinned;
} colimoe_cache_info;
COLIMOE_API size_t colimoe_expert_cache_bytes(const colimoe_config *cfg, int32_t n_slots);
COLIMOE_API size_t colimoe_host_layer_bytes(const colimoe_config *cfg);
COLIMOE_API int colimoe_set_expert_cache(colimoe_ctx *ctx, void *dev, size_t bytes);
COLIMOE_API int colimoe_load_experts_host(colimoe_ctx *ctx, int32_t layer, const colimoe_layer_src *src, void *dev_dst,
                              size_t dev_bytes);
COLIMOE_API int colimoe_cache_set_prefetch(colimoe_ctx *ctx, int32_t depth);
COLIMOE_API int colimoe_cache_repin(colimoe_ctx *ctx, int32_t n);
COLIMOE_API int colimoe_cache_set_autorepin(colimoe_ctx *ctx, int32_t every_tokens, int32_t n);
COLIMOE_API int colimoe_cache_usage(colimoe_ctx *ctx, int32_t layer, uint32_t *counts);
COLIMOE_API int colimoe_cache_usage_save(colimoe_ctx *ctx, const char *path);
COLIMOE_API int colimoe_cache_usage_load(colimoe_ctx *ctx, const char *path);
COLIMOE_API int colimoe_cache_stats(colimoe_ctx *ctx, int64_t *hits, int64_t *misses, int32_t *slots);
COLIMOE_API int colimoe_cache_get_info(colimoe_ctx *ctx, colimoe_cache_info *out);

/* Route T tokens ([A] §1 background: a router picks 8 of the 256 experts of
 * a layer per token; [A] §4: routing is never changed silently, so the
 * selection is deterministic).  Device pointers: x [T][d] fp32 ->
 * logits l[t][e] = sum_c R[e][c] x[t][c] + b[e] in fp32; idx [T][k] int32,
 * the k largest logits, larger first, exact ties to the lower expert id;
 * w [T][k] fp32, the softmax over the k selected logits.  If u is non-NULL
 * its arrays receive the batch-union lists of this routing ([A] §2,
 * batch-union).  logits [T][E] fp32 may be NULL.  Enqueued on the context's
 * stream; allocates nothing.  Errors: E_ARG, E_SHAPE, E_NOT_LOADED,
 * E_WORKSPACE, E_HIP. */
COLIMOE_API int colimoe_route(colimoe_ctx *ctx, int32_t layer, const float *x, int32_t T, int32_t *idx, float *w,
                  const colimoe_union *u, float *logits);

/* Batch-union scheduler on its own ([A] §2, batch-union): builds the union
 * lists of a routing idx [T][k] (device) into u.  An id of -1 marks a slot
 * dropped by expert top-p: it gets no pair (pair_of -1).  A routing with any
 * other id outside [0, E) or an expert twice in one token yields n_unique = 0
 * and makes the next colimoe_sync return E_ARG.  Errors: E_ARG, E_SHAPE,
 * E_WORKSPACE, E_HIP. */
COLIMOE_API int colimoe_union_build(colimoe_ctx *ctx, const int32_t *idx, int32_t T, const colimoe_union *u);

/* The experts of one layer for T tokens: residual[T][d] += MoE(x) under the
 * given routing.  Each routed expert is the three adjacent matrices of [A] §2
 * (gate, up, down; y = Wd (SiLU(Wg x) * (Wu x))), the shared expert runs for
 * every token with weight 1 ([D] §3), and the outputs are added in ascending
 * expert id, then the shared expert.  Batched tokens read each distinct
 * expert from HBM once per call ([A] §2, batch-union); at batch 1 the
 * weights are dequantised to fp32-class arithmetic, for many tokens per
 * expert the grouped bf16 matrix-core path applies ([D] §4, highlight 4).
 * Device pointers: x [T][d] fp32; idx [T][k] int32 and w [T][k] fp32 are
 * inputs, so a caller may force a routing (an id of -1 is a dropped slot,
 * as expert top-p writes it); residual [T][d] fp32, updated in place.  u:
 * union lists for this idx, as written by colimoe_route, or NULL to rebuild
 * them in the workspace.  flags: one of colimoe_forward_flags
 * (no silent change of path, [A] §4: a flag the shapes do not allow is
 * E_SHAPE).  The fp32-class paths give each token bit-identical results
 * whether it runs alone or batched with others.  Errors: E_ARG, E_SHAPE,
 * E_NOT_LOADED, E_WORKSPACE, E_HIP. */
COLIMOE_API int colimoe_forward(colimoe_ctx *ctx, int32_t layer, const float *x, int32_t T, const int32_t *idx,
                    const float *w, const colimoe_union *u, float *residual, uint32_t flags);

/* Adaptive expert top-p ([D] key tuning parameters, "topp=0.7": an adaptive
 * expert top-p that reads 30-40% fewer experts; [D] §4: top-p decides which
 * experts are read).  With p < 1, colimoe_route, colimoe_route_forward and
 * colimoe_rmsnorm_route_forward keep, for each token, of the k selected
 * experts in top-k order, the shortest prefix whose gate weights (softmax
 * over the k) sum to at least p (at least the first one); the kept experts
 * get the softmax over their own logits, and a dropped slot gets idx -1 and
 * weight 0 (pair_of -1 in the union lists, which list the kept experts
 * only), so the layer reads the kept experts and the shared expert only.  A
 * token's result does not depend on the other tokens of the call.  p = 1
 * (the default) is plain top-k.  The setting stays until changed.  Errors:
 * E_ARG (null ctx, p not in (0, 1]). */
COLIMOE_API int colimoe_set_expert_top_p(colimoe_ctx *ctx, float p);

/* colimoe_route followed by colimoe_forward on the same x, as one call: the
 * route kernel also encodes x for the fixed-point path, saving a launch.
 * idx, w (outputs) and u (NULL: the workspace's lists) are written as by
 * colimoe_route.  Errors: as colimoe_route and colimoe_forward. */
COLIMOE_API int colimoe_route_forward(colimoe_ctx *ctx, int32_t layer, const float *x, int32_t T, int32_t *idx, float *w,
                          const colimoe_union *u, float *residual, uint32_t flags);

/* For callers that cannot allocate device memory or hand over a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same computation, arguments and results as
 * colimoe_route_forward (bit for bit), but every scratch buffer the kernels
 * use (logits, union lists when u is NULL, fixed-point encodings, h, y, error
 * word) lives in a fixed device array inside the library, 32 MiB
 * (COLIMOE_STATIC_SCRATCH_BYTES) per device, held by each device the library
 * runs on until the process ends; the context's own workspace is neither
 * needed nor touched.  The call allocates nothing, neither device nor host
 * memory, and creates no events (kernel timing is skipped for it).
 * The array is looked up once per device by colimoe_create, with that device
 * current.
 * Limit: a call whose workspace at this T exceeds the array returns
 * E_WORKSPACE with no effect (at d = 6144, f = 2048, E = 256, k = 8 and a
 * shared expert, calls of up to 63 tokens fit).
 * Sharing: every call on one device uses that device's one array, which
 * keeps the last call's contents (the call clears what must start at zero).
 * Calls that overlap in time on one device (different streams, threads or
 * contexts) race on the array and give undefined results: serialise them.
 * A rejected routing would be reported by the next colimoe_sync, as for the
 * other calls.  Errors: E_ARG, E_SHAPE, E_NOT_LOADED, E_WORKSPACE (this T
 * needs more than the array), E_HIP (the lookup at colimoe_create failed, or
 * a launch failed). */
#define COLIMOE_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
COLIMOE_API int colimoe_route_forward_static(colimoe_ctx *ctx, int32_t layer, const float *x, int32_t T,
                                             int32_t *idx, float *w, const colimoe_union *u, float *residual,
                                             uint32_t flags);

/* x_out[t] = r[t] / sqrt(mean(r[t]^2) + eps), unit weight, fp32 (device
 * pointers, [T][d], 16-byte aligned); lets a stack of layers run without
 * leaving the GPU.  Errors: E_ARG, E_SHAPE, E_HIP. */
COLIMOE_API int colimoe_rmsnorm(colimoe_ctx *ctx, const float *r, int32_t T, float eps, float *x_out);

/* colimoe_rmsnorm(r -> x_out) followed by colimoe_route_forward(x_out, with
 * residual r), as one call: the step of a stack of layers.  r [T][d] is the
 * residual (read, then updated in place: r += MoE(x_out)); x_out [T][d]
 * receives RMSNorm(r) (eps, unit weight); idx, w, u as colimoe_route_forward.
 * For one token on the fixed-point path the router forms x_out on the fly
 * (one launch fewer); the results are those of the two calls bit for bit.
 * Device pointers; r and x_out 16-byte aligned.  Errors: as colimoe_rmsnorm
 * and colimoe_route_forward. */
COLIMOE_API int colimoe_rmsnorm_route_forward(colimoe_ctx *ctx, int32_t layer, float *r, int32_t T, float eps,
                                  float *x_out, int32_t *idx, float *w, const colimoe_union *u, uint32_t flags);

/* One expert on one token through the fp32 path, every stage exposed
 * (device pointers, any of g/u/h may be NULL): x [d] -> g, u, h [f], y [d].
 * e = -1 selects the shared expert.  Debug and parity only. */
COLIMOE_API int colimoe_debug_expert(colimoe_ctx *ctx, int32_t layer, int32_t e, const float *x, float *g, float *u,
                         float *h, float *y);

/* Per-kernel timing for measurement.  While enabled, every kernel launch of
 * the context is bracketed by a pair of HIP events on its stream (this adds
 * two event records per launch).  Kernel names: "route" (router; in
 * colimoe_route_forward with T <= 16 it also encodes x), "topk" (top-k; with
 * the union lists when T == 1), "union", "encode" (fixed-point encoding of x,
 * or the M-block list and bf16 gather of the MFMA path), "gateup", "down"
 * (with the combine when T == 1 or when it fits in LDS), "combine",
 * "rmsnorm". */
COLIMOE_API int colimoe_timing_enable(colimoe_ctx *ctx, int enable);

/* Synchronises the stream, then reports the summed duration (ms) and the
 * number of launches of kernel `name` recorded since the last reset; clears
 * the records if reset != 0.  Errors: E_ARG (unknown name), E_HIP. */
COLIMOE_API int colimoe_timing_read(colimoe_ctx *ctx, const char *name, double *total_ms, int64_t *count, int reset);

/* Wait for the context's stream; reports a kernel fault as E_HIP. */
COLIMOE_API int colimoe_sync(colimoe_ctx *ctx);

/* Static text for a status code. */
COLIMOE_API const char *colimoe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* COLIMOE_H */
