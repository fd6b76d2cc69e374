// cache.cpp - tiered placement of routed experts: layers whose experts stay
// in pinned host memory, served through an HBM cache of expert slots.
//
// Sources, cited by page title and section:
//   [A] "Colibrì: running a 744B MoE model on a laptop with 2400 lines of pure C"
//       (kechuai.cn article)
//   [D] "colibrì: 1300 lines of C, a 25 GB laptop, a 744-billion-parameter model"
//       (SSP GitHub Daily #091, jsqmd.com)
//
// What the pages describe ([A] §2; [D] §3 and key tuning parameters): the
// routed experts are data moved between storage tiers by how often routing
// asks for them; each layer keeps a least-recently-used cache of experts;
// the engine records which experts the workload routes to and keeps the
// hottest pinned (a learned hot set saved between runs), re-placed every N
// tokens; and the router of the next layer runs one layer ahead on the
// current input, so that the experts it predicts are already on their way
// when the next layer needs them.  Here pinned host memory plays the disk,
// PCIe the NVMe link and HBM the RAM.
//
// Layer l owns slots [l * per_layer, (l + 1) * per_layer) of the cache, its
// shared expert fixed in the first one.  A call brings its misses into the
// least recently used evictable slots of its own layer, so a layer's calls
// never evict another layer's experts.  Results do not depend on the cache:
// the kernels read each expert through the layer's slot map, so a
// host-resident layer gives the bits of the same layer resident in HBM.
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "context.h"

using namespace colimoe;

namespace colimoe {

namespace {

constexpr char kUsageMagic[8] = {'C', 'O', 'L', 'I', 'U', 'S', 'E', '1'};
constexpr int kPredMaxT = kRouteSplitMaxT;  // predictions for calls of up to this many tokens

struct CacheLayout {
  size_t maps, pred_logits, pred_idx, pred_w, slots;
};

CacheLayout cache_layout(const colimoe_config *c) {
  CacheLayout L;
  size_t o = 0;
  L.maps = o;
  o += align_up((size_t)c->n_layers * (c->n_experts + 1) * 4, kAlign);
  L.pred_logits = o;
  o += align_up((size_t)kPredMaxT * c->n_experts * 4, kAlign);
  L.pred_idx = o;
  o += align_up((size_t)kPredMaxT * c->top_k * 4, kAlign);
  L.pred_w = o;
  o += align_up((size_t)kPredMaxT * c->top_k * 4, kAlign);
  L.slots = o;
  return L;
}

int part_begin(const ExpertCache &C, int l) { return l * C.per_layer; }

// Slot of the least recently used evictable slot of layer l whose stamp is
// not `now` (those hold experts the current operation needs), or -1.
int lru_victim(const ExpertCache &C, int l, uint64_t now) {
  int v = -1;
  const int b = part_begin(C, l);
  for (int i = b; i < b + C.per_layer; ++i)
    if (!C.fixed[i] && C.used[i] != now && (v < 0 || C.used[i] < C.used[v])) v = i;
  return v;
}

// Slot i now holds expert e of layer l (whatever it held is forgotten).
void assign(ExpertCache &C, int E, int l, int i, int e) {
  if (C.tag[i] >= 0) C.slot_of[(size_t)l * (E + 1) + C.tag[i]] = -1;
  C.tag[i] = e;
  C.slot_of[(size_t)l * (E + 1) + e] = i;
  C.fresh[i] = 0;
}

// Uploads layer l's slot map: an expert not in the cache points at the
// layer's first slot, so every address a kernel forms stays inside the cache.
int upload_map(colimoe_ctx *ctx, int l, hipStream_t s) {
  ExpertCache &C = ctx->cache;
  const int E = ctx->cfg.n_experts;
  const int32_t *map = &C.slot_of[(size_t)l * (E + 1)];
  int32_t *st = C.stage + (size_t)l * (E + 1);
  const int dummy = part_begin(C, l);
  for (int e = 0; e <= E; ++e) st[e] = map[e] >= 0 ? map[e] : dummy;
  return hip_status(
      hipMemcpyAsync(C.dev_maps + (size_t)l * (E + 1), st, (size_t)(E + 1) * 4, hipMemcpyHostToDevice, s));
}

// Orders stream s after the prefetch copy into slot i, if one may still run
// (before the slot is read, or overwritten by a copy on another stream).
int wait_slot(ExpertCache &C, int i, hipStream_t s) {
  if (!C.pending[i]) return COLIMOE_OK;
  C.pending[i] = 0;
  return hip_status(hipStreamWaitEvent(s, C.ev_slot[i], 0));
}

// Waits on the host for every prefetch copy into layer l's partition.
int settle_layer(ExpertCache &C, int l) {
  bool any = false;
  const int b = part_begin(C, l);
  for (int i = b; i < b + C.per_layer; ++i) {
    any = any || C.pending[i];
    C.pending[i] = 0;
  }
  return any ? hip_status(hipStreamSynchronize(C.copy)) : COLIMOE_OK;
}

// Learned pinning of one layer: its n experts with the largest usage counts
// (ties to the lower id) are pinned in its partition, loading the absent
// ones; the rest of its experts become evictable.  Runs with no kernel
// reading the layer's slots (the caller synchronised the stream).
int repin_layer(colimoe_ctx *ctx, int l, int n) {
  ExpertCache &C = ctx->cache;
  const int E = ctx->cfg.n_experts;
  const size_t be = ctx->el.bytes;
  hipStream_t s = ctx->stream;
  int rc = settle_layer(C, l);
  if (rc) return rc;
  std::vector<int> cand;
  for (int e = 0; e < E; ++e)
    if (C.uses[(size_t)l * E + e]) cand.push_back(e);
  std::stable_sort(cand.begin(), cand.end(),
                   [&](int a, int b) { return C.uses[(size_t)l * E + a] > C.uses[(size_t)l * E + b]; });
  if ((int)cand.size() > n) cand.resize(n);
  const int b = part_begin(C, l);
  for (int i = b; i < b + C.per_layer; ++i)
    if (C.fixed[i] == 2) C.fixed[i] = 0;
  const int32_t *map = &C.slot_of[(size_t)l * (E + 1)];
  for (int e : cand)
    if (map[e] >= 0) C.fixed[map[e]] = 2;
  const uint64_t now = ++C.stamp;
  for (int e : cand) {
    if (map[e] >= 0) continue;
    const int v = lru_victim(C, l, now);
    if (v < 0) return COLIMOE_E_WORKSPACE;
    if (hipMemcpyAsync(C.slots + (size_t)v * be, ctx->host_store[l] + (size_t)e * be, be, hipMemcpyHostToDevice,
                       s) != hipSuccess)
      return COLIMOE_E_HIP;
    assign(C, E, l, v, e);
    C.used[v] = now;
    C.fixed[v] = 2;
  }
  return upload_map(ctx, l, s);
}

int max_pinned(const colimoe_ctx *ctx) {
  return ctx->cache.per_layer - ctx->cfg.n_shared - ctx->cfg.top_k;  // one token's experts must still fit
}

}  // namespace

int cache_ensure_resident(colimoe_ctx *ctx, int l, const int32_t *idx, int T) {
  ExpertCache &C = ctx->cache;
  const int E = ctx->cfg.n_experts, k = ctx->cfg.top_k;
  const size_t be = ctx->el.bytes;
  hipStream_t s = ctx->stream;
  if (hipMemcpyAsync(C.idx_host, idx, (size_t)T * k * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return COLIMOE_E_HIP;
  std::vector<int> need;
  for (int i = 0; i < T * k; ++i) {
    const int e = C.idx_host[i];
    if (e >= 0 && e < E) {
      need.push_back(e);
      C.uses[(size_t)l * E + e] += 1;  // usage histogram: tokens routed to e
    }
  }
  std::sort(need.begin(), need.end());
  need.erase(std::unique(need.begin(), need.end()), need.end());
  // how many of this call's experts the one-layer-ahead prediction named
  if (!C.pred[l].empty()) {
    for (int e : need) {
      ++C.predicted;
      C.predicted_hits += std::binary_search(C.pred[l].begin(), C.pred[l].end(), e);
    }
    C.pred[l].clear();
  }
  // automatic learned pinning, every repin_every tokens of this layer
  C.tokens[l] += T;
  if (C.repin_every > 0 && C.tokens[l] >= C.repin_every) {
    C.tokens[l] = 0;
    const int rc = repin_layer(ctx, l, std::min(C.repin_n, max_pinned(ctx)));
    if (rc) return rc;
  }
  // the call's experts that must sit in evictable slots: the misses, and the
  // hits that already sit in one (a pinned or shared slot is not evictable)
  int32_t *map = &C.slot_of[(size_t)l * (E + 1)];
  const int b = part_begin(C, l);
  int free_slots = 0, want_free = 0;
  for (int i = b; i < b + C.per_layer; ++i) free_slots += !C.fixed[i];
  for (int e : need) want_free += map[e] < 0 || !C.fixed[map[e]];
  if (want_free > free_slots) return COLIMOE_E_WORKSPACE;
  const uint64_t now = ++C.stamp;
  for (int e : need)
    if (map[e] >= 0) {
      const int i = map[e];
      C.used[i] = now;
      ++C.hits;
      if (C.fresh[i]) {
        ++C.prefetched_used;
        C.fresh[i] = 0;
      }
      const int rc = wait_slot(C, i, s);  // a predicted expert still on its way
      if (rc) return rc;
    }
  for (int e : need) {
    if (map[e] >= 0) continue;
    const int v = lru_victim(C, l, now);
    if (v < 0) return COLIMOE_E_WORKSPACE;
    const int rc = wait_slot(C, v, s);  // an unused prediction still being copied in
    if (rc) return rc;
    if (hipMemcpyAsync(C.slots + (size_t)v * be, ctx->host_store[l] + (size_t)e * be, be, hipMemcpyHostToDevice,
                       s) != hipSuccess)
      return COLIMOE_E_HIP;
    assign(C, E, l, v, e);
    C.used[v] = now;
    ++C.misses;
  }
  return upload_map(ctx, l, s);
}

int cache_predict_start(colimoe_ctx *ctx, int l, const float *x, int T) {
  ExpertCache &C = ctx->cache;
  const int nl = l + 1;
  if (C.prefetch <= 0 || nl >= ctx->cfg.n_layers || !ctx->host_store[nl] || !ctx->loaded[nl] || T > kPredMaxT)
    return 0;
  // layer nl's router and top-k on this call's input, on the side stream; the
  // caller's stream was synchronised by cache_ensure_resident, so x is ready
  // and the prediction runs beside this layer's expert kernels
  const Dims D = dims_of(ctx, T);
  if (launch_router_split(ctx->layers[nl], D, x, C.pred_logits, nullptr, nullptr, C.side) != hipSuccess ||
      launch_topk(C.pred_logits, D, C.pred_idx, C.pred_w, 1.0f, C.side) != hipSuccess ||
      hipMemcpyAsync(C.pred_host, C.pred_idx, (size_t)T * ctx->cfg.top_k * 4, hipMemcpyDeviceToHost, C.side) !=
          hipSuccess)
    return COLIMOE_E_HIP;
  return 1;
}

int cache_prefetch_issue(colimoe_ctx *ctx, int l, int T) {
  ExpertCache &C = ctx->cache;
  const int nl = l + 1;
  const int E = ctx->cfg.n_experts, k = ctx->cfg.top_k;
  const size_t be = ctx->el.bytes;
  if (hipStreamSynchronize(C.side) != hipSuccess) return COLIMOE_E_HIP;  // the prediction only
  // the predicted experts (all k per token count for the hit rate); the first
  // `prefetch` of each token's prediction (its largest logits) are fetched
  std::vector<int32_t> P, F;
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      const int e = C.pred_host[t * k + j];
      if (e < 0 || e >= E) continue;
      P.push_back(e);
      if (j < C.prefetch) F.push_back(e);
    }
  std::sort(P.begin(), P.end());
  P.erase(std::unique(P.begin(), P.end()), P.end());
  C.pred[nl] = P;
  std::sort(F.begin(), F.end());
  F.erase(std::unique(F.begin(), F.end()), F.end());
  // copy the predicted misses into layer nl's least recently used evictable
  // slots.  No kernel reads them now: layer nl's last calls finished before
  // this call's routing was read on the host, and its next call orders
  // itself after these copies.
  const int32_t *map = &C.slot_of[(size_t)nl * (E + 1)];
  const uint64_t now = ++C.stamp;
  for (int e : F) {
    if (map[e] >= 0) continue;
    const int v = lru_victim(C, nl, now);
    if (v < 0) break;
    // a slot still receiving an earlier prefetch is overwritten in stream order
    if (hipMemcpyAsync(C.slots + (size_t)v * be, ctx->host_store[nl] + (size_t)e * be, be, hipMemcpyHostToDevice,
                       C.copy) != hipSuccess ||
        hipEventRecord(C.ev_slot[v], C.copy) != hipSuccess)
      return COLIMOE_E_HIP;
    assign(C, E, nl, v, e);
    C.used[v] = now;
    C.fresh[v] = 1;
    C.pending[v] = 1;
    ++C.prefetched;
  }
  return COLIMOE_OK;
}

void cache_drop_layer(colimoe_ctx *ctx, int l) {
  ExpertCache &C = ctx->cache;
  const int E = ctx->cfg.n_experts;
  if (C.slots) {
    (void)settle_layer(C, l);
    const int b = part_begin(C, l);
    for (int i = b; i < b + C.per_layer; ++i) {
      C.tag[i] = -1;
      C.used[i] = 0;
      C.fixed[i] = 0;
      C.fresh[i] = 0;
    }
    for (int e = 0; e <= E; ++e) C.slot_of[(size_t)l * (E + 1) + e] = -1;
    for (int e = 0; e < E; ++e) C.uses[(size_t)l * E + e] = 0;
    C.tokens[l] = 0;
    C.pred[l].clear();
  }
  if (ctx->host_store[l]) {
    (void)hipHostFree(ctx->host_store[l]);
    ctx->host_store[l] = nullptr;
  }
}

void cache_release(colimoe_ctx *ctx) {
  ExpertCache &C = ctx->cache;
  if (C.copy) (void)hipStreamSynchronize(C.copy);
  if (C.side) (void)hipStreamSynchronize(C.side);
  for (hipEvent_t e : C.ev_slot)
    if (e) (void)hipEventDestroy(e);
  C.ev_slot.clear();
  if (C.copy) (void)hipStreamDestroy(C.copy);
  if (C.side) (void)hipStreamDestroy(C.side);
  C.copy = C.side = nullptr;
  for (int32_t *p : {C.stage, C.idx_host, C.pred_host})
    if (p) (void)hipHostFree(p);
  C.stage = C.idx_host = C.pred_host = nullptr;
  for (uint8_t *&h : ctx->host_store)
    if (h) {
      (void)hipHostFree(h);
      h = nullptr;
    }
}

}  // namespace colimoe

extern "C" {

size_t colimoe_host_layer_bytes(const colimoe_config *cfg) {
  if (!cfg_ok(cfg)) return 0;
  return router_bytes(cfg);
}

size_t colimoe_expert_cache_bytes(const colimoe_config *cfg, int32_t n_slots) {
  if (!cfg_ok(cfg) || n_slots < 1) return 0;
  return cache_layout(cfg).slots + (size_t)n_slots * cfg_expert_bytes(cfg);
}

int colimoe_set_expert_cache(colimoe_ctx *ctx, void *dev, size_t bytes) {
  if (!ctx || !dev || !aligned(dev, kAlign)) return COLIMOE_E_ARG;
  for (uint8_t *h : ctx->host_store)
    if (h) return COLIMOE_E_STATE;  // the cache cannot move under host-resident layers
  const colimoe_config *c = &ctx->cfg;
  const CacheLayout CL = cache_layout(c);
  const size_t be = ctx->el.bytes;
  if (bytes < CL.slots + be) return COLIMOE_E_WORKSPACE;
  ExpertCache &C = ctx->cache;
  const int L = c->n_layers, E = c->n_experts;
  if (!C.stage && hipHostMalloc((void **)&C.stage, (size_t)L * (E + 1) * 4, hipHostMallocDefault) != hipSuccess)
    return COLIMOE_E_HIP;
  if (!C.idx_host &&
      hipHostMalloc((void **)&C.idx_host, (size_t)c->max_tokens * c->top_k * 4, hipHostMallocDefault) != hipSuccess)
    return COLIMOE_E_HIP;
  if (!C.pred_host &&
      hipHostMalloc((void **)&C.pred_host, (size_t)kPredMaxT * c->top_k * 4, hipHostMallocDefault) != hipSuccess)
    return COLIMOE_E_HIP;
  if (!C.copy && hipStreamCreateWithFlags(&C.copy, hipStreamNonBlocking) != hipSuccess) return COLIMOE_E_HIP;
  if (!C.side && hipStreamCreateWithFlags(&C.side, hipStreamNonBlocking) != hipSuccess) return COLIMOE_E_HIP;
  uint8_t *base = (uint8_t *)dev;
  C.dev_maps = (int32_t *)(base + CL.maps);
  C.pred_logits = (float *)(base + CL.pred_logits);
  C.pred_idx = (int32_t *)(base + CL.pred_idx);
  C.pred_w = (float *)(base + CL.pred_w);
  C.slots = base + CL.slots;
  C.n_slots = (int)std::min<size_t>((bytes - CL.slots) / be, (size_t)1 << 30);
  if (C.copy && hipStreamSynchronize(C.copy) != hipSuccess) return COLIMOE_E_HIP;
  while ((int)C.ev_slot.size() < C.n_slots) {
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return COLIMOE_E_HIP;
    C.ev_slot.push_back(e);
  }
  C.per_layer = C.n_slots / L;
  C.slot_of.assign((size_t)L * (E + 1), -1);
  C.tag.assign(C.n_slots, -1);
  C.used.assign(C.n_slots, 0);
  C.fixed.assign(C.n_slots, 0);
  C.fresh.assign(C.n_slots, 0);
  C.uses.assign((size_t)L * E, 0);
  C.tokens.assign(L, 0);
  C.pred.assign(L, {});
  C.pending.assign(C.n_slots, 0);
  C.stamp = 0;
  C.hits = C.misses = C.predicted = C.predicted_hits = C.prefetched = C.prefetched_used = 0;
  return COLIMOE_OK;
}

int colimoe_load_experts_host(colimoe_ctx *ctx, int32_t layer, const colimoe_layer_src *src, void *dev_dst,
                              size_t dev_bytes) {
  if (!ctx || !src || !dev_dst || !src->router || !src->experts) return COLIMOE_E_ARG;
  const colimoe_config *c = &ctx->cfg;
  if (layer < 0 || layer >= c->n_layers) return COLIMOE_E_SHAPE;
  if ((c->n_shared == 1) != (src->shared != nullptr)) return COLIMOE_E_ARG;
  if (!aligned(dev_dst, kAlign)) return COLIMOE_E_ARG;
  if (dev_bytes < router_bytes(c)) return COLIMOE_E_SHAPE;
  ExpertCache &C = ctx->cache;
  if (!C.slots) return COLIMOE_E_STATE;  // colimoe_set_expert_cache first
  if (C.per_layer < c->n_shared + c->top_k) return COLIMOE_E_WORKSPACE;  // room for one token's experts
  const int E = c->n_experts;
  const size_t be = ctx->el.bytes;
  hipStream_t s = ctx->stream;
  if (hipStreamSynchronize(s) != hipSuccess) return COLIMOE_E_HIP;  // no kernel still reads the layer
  ctx->loaded[layer] = 0;
  cache_drop_layer(ctx, layer);
  float *router = (float *)dev_dst;
  float *bias = (float *)((uint8_t *)dev_dst + align_up((size_t)E * c->d * 4, kAlign));
  if (hipMemcpyAsync(router, src->router, (size_t)E * c->d * 4, hipMemcpyHostToDevice, s) != hipSuccess)
    return COLIMOE_E_HIP;
  if (src->bias) {
    if (hipMemcpyAsync(bias, src->bias, (size_t)E * 4, hipMemcpyHostToDevice, s) != hipSuccess) return COLIMOE_E_HIP;
  } else if (hipMemsetAsync(bias, 0, (size_t)E * 4, s) != hipSuccess) {
    return COLIMOE_E_HIP;
  }
  uint8_t *store = nullptr;
  if (hipHostMalloc((void **)&store, (size_t)E * be, hipHostMallocDefault) != hipSuccess) return COLIMOE_E_HIP;
  std::vector<const uint8_t *> srcs(E);
  for (int e = 0; e < E; ++e) srcs[e] = src->experts + (size_t)e * be;
  if (c->flags & COLIMOE_CFG_INT8)
    copy_many(srcs.data(), store, E, be);
  else
    repack_many(srcs.data(), store, E, be, c->d, c->f);
  if (c->n_shared) {  // the shared expert: the first slot of the layer's partition, for the layer's lifetime
    uint8_t *tmp = nullptr;
    if (hipHostMalloc((void **)&tmp, be, hipHostMallocDefault) != hipSuccess) {
      (void)hipHostFree(store);
      return COLIMOE_E_HIP;
    }
    if (c->flags & COLIMOE_CFG_INT8)
      memcpy(tmp, src->shared, be);
    else
      repack_expert(src->shared, tmp, c->d, c->f);
    const int i = part_begin(C, layer);
    const bool ok = hipMemcpyAsync(C.slots + (size_t)i * be, tmp, be, hipMemcpyHostToDevice, s) == hipSuccess &&
                    hipStreamSynchronize(s) == hipSuccess;
    (void)hipHostFree(tmp);
    if (!ok) {
      (void)hipHostFree(store);
      return COLIMOE_E_HIP;
    }
    assign(C, E, layer, i, E);
    C.fixed[i] = 1;
  }
  if (upload_map(ctx, layer, s) != COLIMOE_OK || hipStreamSynchronize(s) != hipSuccess) {
    (void)hipHostFree(store);
    return COLIMOE_E_HIP;
  }
  ctx->host_store[layer] = store;
  ctx->layers[layer] = LayerDev{router, bias, C.slots, be, C.dev_maps + (size_t)layer * (E + 1)};
  ctx->loaded[layer] = 1;
  return COLIMOE_OK;
}

int colimoe_cache_repin(colimoe_ctx *ctx, int32_t n) {
  if (!ctx || n < 0) return COLIMOE_E_ARG;
  ExpertCache &C = ctx->cache;
  if (!C.slots) return COLIMOE_E_STATE;
  if (n > max_pinned(ctx)) return COLIMOE_E_WORKSPACE;
  if (hipStreamSynchronize(ctx->stream) != hipSuccess) return COLIMOE_E_HIP;  // no kernel still reads a slot
  for (int l = 0; l < ctx->cfg.n_layers; ++l)
    if (ctx->host_store[l]) {
      const int rc = repin_layer(ctx, l, n);
      if (rc) return rc;
    }
  return hip_status(hipStreamSynchronize(ctx->stream));
}

int colimoe_cache_set_autorepin(colimoe_ctx *ctx, int32_t every_tokens, int32_t n) {
  if (!ctx || every_tokens < 0 || n < 0) return COLIMOE_E_ARG;
  ExpertCache &C = ctx->cache;
  if (!C.slots) return COLIMOE_E_STATE;
  if (every_tokens > 0 && n > max_pinned(ctx)) return COLIMOE_E_WORKSPACE;
  C.repin_every = every_tokens;
  C.repin_n = n;
  std::fill(C.tokens.begin(), C.tokens.end(), 0);
  return COLIMOE_OK;
}

int colimoe_cache_set_prefetch(colimoe_ctx *ctx, int32_t depth) {
  if (!ctx || depth < 0 || depth > ctx->cfg.top_k) return COLIMOE_E_ARG;
  if (!ctx->cache.slots) return COLIMOE_E_STATE;
  ctx->cache.prefetch = depth;
  return COLIMOE_OK;
}

int colimoe_cache_stats(colimoe_ctx *ctx, int64_t *hits, int64_t *misses, int32_t *slots) {
  if (!ctx || !hits || !misses || !slots) return COLIMOE_E_ARG;
  *hits = ctx->cache.hits;
  *misses = ctx->cache.misses;
  *slots = ctx->cache.n_slots;
  return COLIMOE_OK;
}

int colimoe_cache_get_info(colimoe_ctx *ctx, colimoe_cache_info *out) {
  if (!ctx || !out) return COLIMOE_E_ARG;
  const ExpertCache &C = ctx->cache;
  out->hits = C.hits;
  out->misses = C.misses;
  out->predicted = C.predicted;
  out->predicted_hits = C.predicted_hits;
  out->prefetched = C.prefetched;
  out->prefetched_used = C.prefetched_used;
  out->slots = C.n_slots;
  out->slots_per_layer = C.per_layer;
  int pinned = 0;
  for (char f : C.fixed) pinned += f == 2;
  out->pinned = pinned;
  return COLIMOE_OK;
}

int colimoe_cache_usage(colimoe_ctx *ctx, int32_t layer, uint32_t *counts) {
  if (!ctx || !counts) return COLIMOE_E_ARG;
  if (layer < 0 || layer >= ctx->cfg.n_layers) return COLIMOE_E_SHAPE;
  if (!ctx->cache.slots) return COLIMOE_E_STATE;
  const int E = ctx->cfg.n_experts;
  memcpy(counts, &ctx->cache.uses[(size_t)layer * E], (size_t)E * 4);
  return COLIMOE_OK;
}

int colimoe_cache_usage_save(colimoe_ctx *ctx, const char *path) {
  if (!ctx || !path) return COLIMOE_E_ARG;
  const ExpertCache &C = ctx->cache;
  if (!C.slots) return COLIMOE_E_STATE;
  FILE *f = fopen(path, "wb");
  if (!f) return COLIMOE_E_ARG;
  const int32_t dims[2] = {ctx->cfg.n_layers, ctx->cfg.n_experts};
  bool ok = fwrite(kUsageMagic, 1, 8, f) == 8 && fwrite(dims, 4, 2, f) == 2 &&
            fwrite(C.uses.data(), 4, C.uses.size(), f) == C.uses.size();
  ok = (fclose(f) == 0) && ok;
  return ok ? COLIMOE_OK : COLIMOE_E_ARG;
}

int colimoe_cache_usage_load(colimoe_ctx *ctx, const char *path) {
  if (!ctx || !path) return COLIMOE_E_ARG;
  ExpertCache &C = ctx->cache;
  if (!C.slots) return COLIMOE_E_STATE;
  FILE *f = fopen(path, "rb");
  if (!f) return COLIMOE_E_ARG;
  char magic[8];
  int32_t dims[2];
  std::vector<uint32_t> u(C.uses.size());
  const bool header = fread(magic, 1, 8, f) == 8 && memcmp(magic, kUsageMagic, 8) == 0 && fread(dims, 4, 2, f) == 2;
  const bool shape = header && dims[0] == ctx->cfg.n_layers && dims[1] == ctx->cfg.n_experts;
  const bool body = shape && fread(u.data(), 4, u.size(), f) == u.size();
  fclose(f);
  if (!header) return COLIMOE_E_ARG;   // not a usage file
  if (!shape) return COLIMOE_E_SHAPE;  // another model's layers or experts
  if (!body) return COLIMOE_E_ARG;     // truncated
  C.uses = u;
  return COLIMOE_OK;
}

}  // extern "C"
