// host.cpp - C ABI of the int4 routed-expert MoE layer (include/colimoe.h):
// argument validation, workspace carve-up, the layer loader (canonical blobs
// -> device layout) and kernel sequencing.  Sources are cited by page title
// and section:
//   [A] "Colibrì: running a 744B MoE model on a laptop with 2400 lines of pure C"
//       (kechuai.cn article)
//   [P] "colibrì" project profile (gh.puless.com)
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "context.h"

using namespace colimoe;


namespace {
// "route": the fused route kernel, or the router GEMV/GEMM when top-k runs apart.
const char *const kKernelNames[] = {"route", "topk", "union", "encode", "gateup", "down", "combine", "rmsnorm"};
enum { K_ROUTE, K_TOPK, K_UNION, K_ENCODE, K_GATEUP, K_DOWN, K_COMBINE, K_RMSNORM, K_COUNT };

// Timing events skip the system-scope fence (cache write-back and
// invalidation) at each record: they only time, and their readout
// synchronises the stream first.
hipEvent_t take_event(colimoe_ctx *c) {
  if (c->ev_used == c->ev_pool.size()) {
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    c->ev_pool.push_back(e);
  }
  return c->ev_pool[c->ev_used++];
}

// Brackets one kernel launch with events when timing is on.
struct KTimer {
  colimoe_ctx *c;
  int kid;
  hipEvent_t a = nullptr;
  KTimer(colimoe_ctx *c_, int kid_) : c(c_), kid(kid_) {
    if (c->timing && (a = take_event(c))) (void)hipEventRecord(a, c->stream);
  }
  ~KTimer() {
    if (!a) return;
    hipEvent_t b = take_event(c);
    if (!b) return;
    (void)hipEventRecord(b, c->stream);
    c->recs.push_back({kid, a, b});
  }
};

int drain_timing(colimoe_ctx *c) {
  if (c->recs.empty()) return COLIMOE_OK;
  if (hipStreamSynchronize(c->stream) != hipSuccess) return COLIMOE_E_HIP;
  for (auto &r : c->recs) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return COLIMOE_E_HIP;
    c->tot_ms[r.kid] += ms;
    c->cnt[r.kid] += 1;
  }
  c->recs.clear();
  c->ev_used = 0;
  return COLIMOE_OK;
}
}  // namespace

namespace colimoe {

bool cfg_ok(const colimoe_config *c) {
  if (!c) return false;
  if (c->d <= 0 || c->f <= 0 || c->d % kGroup || c->f % kGroup) return false;
  if (c->d > 16384 || c->f > 16384) return false;  // gate/up: at most 8 waves of 64 chunks per tile
  if (c->n_experts < 1 || c->n_experts > 1024) return false;
  if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->n_experts) return false;
  if (c->n_layers < 1 || c->n_shared < 0 || c->n_shared > 1) return false;
  if (c->group_size != kGroup) return false;
  if (c->max_tokens < 1 || c->max_tokens > 65536) return false;
  if ((long long)c->max_tokens * c->top_k > (1LL << 24)) return false;
  if (c->flags & ~(uint32_t)COLIMOE_CFG_INT8) return false;
  return true;
}

// Bytes of one expert in the context's container (int4 device layout, or the
// int8 canonical layout).
size_t cfg_expert_bytes(const colimoe_config *c) {
  return (c->flags & COLIMOE_CFG_INT8) ? expert_bytes_i8(c->d, c->f) : expert_layout(c->d, c->f).bytes;
}

size_t router_bytes(const colimoe_config *c) {
  return align_up((size_t)c->n_experts * c->d * 4, kAlign) + align_up((size_t)c->n_experts * 4, kAlign);
}

Dims dims_of(const colimoe_ctx *ctx, int T) {
  Dims D;
  D.d = ctx->cfg.d;
  D.f = ctx->cfg.f;
  D.E = ctx->cfg.n_experts;
  D.k = ctx->cfg.top_k;
  D.T = T;
  D.n_shared = ctx->cfg.n_shared;
  return D;
}

}  // namespace colimoe

namespace {

LayerDev layer_of(colimoe_ctx *ctx, int layer) { return ctx->layers[layer]; }

UnionDev ws_union(colimoe_ctx *ctx) {
  UnionDev U;
  U.n_unique = (int32_t *)(ctx->ws + ctx->wl.n_unique);
  U.ids = (int32_t *)(ctx->ws + ctx->wl.ids);
  U.offsets = (int32_t *)(ctx->ws + ctx->wl.offsets);
  U.pair_token = (int32_t *)(ctx->ws + ctx->wl.pair_token);
  U.pair_slot = (int32_t *)(ctx->ws + ctx->wl.pair_slot);
  U.pair_of = (int32_t *)(ctx->ws + ctx->wl.pair_of);
  return U;
}

bool union_ok(const colimoe_union *u) {
  return u && u->n_unique && u->ids && u->offsets && u->pair_token && u->pair_slot && u->pair_of &&
         aligned(u->n_unique, 4) && aligned(u->ids, 4) && aligned(u->offsets, 4) && aligned(u->pair_token, 4) &&
         aligned(u->pair_slot, 4) && aligned(u->pair_of, 4);
}

UnionDev to_dev(const colimoe_union *u) {
  UnionDev U;
  U.n_unique = u->n_unique;
  U.ids = u->ids;
  U.offsets = u->offsets;
  U.pair_token = u->pair_token;
  U.pair_slot = u->pair_slot;
  U.pair_of = u->pair_of;
  return U;
}

// Common checks of route/forward/debug: context, layer, workspace, T.
int check_call(colimoe_ctx *ctx, int32_t layer, int32_t T) {
  if (!ctx) return COLIMOE_E_ARG;
  if (layer < 0 || layer >= ctx->cfg.n_layers) return COLIMOE_E_SHAPE;
  if (T < 0 || T > ctx->cfg.max_tokens) return COLIMOE_E_SHAPE;
  if (!ctx->loaded[layer]) return COLIMOE_E_NOT_LOADED;
  if (!ctx->ws) return COLIMOE_E_WORKSPACE;
  return COLIMOE_OK;
}

}  // namespace

namespace colimoe {

// ---------------------------------------------------------------- repacking
// Canonical blob -> device layout (internal.h): gate/up rows interleaved in
// tiles of 4+4, nibbles of a tile stored step-major, scales regrouped per
// (tile, group) so one 16-byte load gives a tile's 8 rows their scale.

// Copies one canonical row of K nibbles into tile row r of tile `tile` of a
// device matrix (step-major tiles).
static inline void put_row(uint8_t *dst_nib, const uint8_t *src_row, int tile, int r, int K) {
  const int C = K / kChunk;
  for (int c0 = 0; c0 < C; c0 += 64) {
    const int width = std::min(64, C - c0);
    memcpy(dst_nib + chunk_offset(tile, K, c0, r), src_row + (size_t)c0 * 16, (size_t)width * 16);
  }
}

void repack_expert(const uint8_t *src, uint8_t *dst, int d, int f) {
  const size_t w = (size_t)d * f, nb = w / 2, ns = w / kGroup;  // bytes of nibbles, number of scales
  const uint8_t *gn = src;
  const uint16_t *gs = (const uint16_t *)(gn + nb);
  const uint8_t *un = gn + nb + 2 * ns;
  const uint16_t *us = (const uint16_t *)(un + nb);
  const uint8_t *dn = un + nb + 2 * ns;
  const uint16_t *ds = (const uint16_t *)(dn + nb);
  const ExpertLayout L = expert_layout(d, f);
  const size_t rowd = (size_t)d / 2, rowf = (size_t)f / 2;
  const int Gd = d / kGroup, Gf = f / kGroup;
  uint16_t *gus = (uint16_t *)(dst + L.gu_sc);
  for (int ti = 0; ti < f / 4; ++ti) {
    for (int r = 0; r < 8; ++r) {
      const int srow = 4 * ti + (r & 3);
      put_row(dst + L.gu_nib, (r < 4 ? gn : un) + (size_t)srow * rowd, ti, r, d);
      const uint16_t *sc = (r < 4 ? gs : us) + (size_t)srow * Gd;
      for (int g = 0; g < Gd; ++g) gus[((size_t)ti * Gd + g) * 8 + r] = sc[g];
    }
  }
  uint16_t *dss = (uint16_t *)(dst + L.dn_sc);
  for (int ti = 0; ti < d / 8; ++ti)
    for (int r = 0; r < 8; ++r) {
      put_row(dst + L.dn_nib, dn + ((size_t)ti * 8 + r) * rowf, ti, r, f);
      for (int g = 0; g < Gf; ++g) dss[((size_t)ti * Gf + g) * 8 + r] = ds[((size_t)ti * 8 + r) * Gf + g];
    }
}

// int8 container: the device layout is the canonical one.
void copy_many(const uint8_t *const *srcs, uint8_t *dst, int n, size_t be) {
  for (int i = 0; i < n; ++i) memcpy(dst + (size_t)i * be, srcs[i], be);
}

void repack_many(const uint8_t *const *srcs, uint8_t *dst, int n, size_t be, int d, int f) {
  unsigned hw = std::thread::hardware_concurrency();
  int nt = (int)std::min<unsigned>(hw ? hw : 4, 16);
  nt = std::min(nt, n);
  if (nt <= 1) {
    for (int i = 0; i < n; ++i) repack_expert(srcs[i], dst + (size_t)i * be, d, f);
    return;
  }
  std::vector<std::thread> th;
  for (int t = 0; t < nt; ++t)
    th.emplace_back([=]() {
      for (int i = t; i < n; i += nt) repack_expert(srcs[i], dst + (size_t)i * be, d, f);
    });
  for (auto &x : th) x.join();
}

Workspace workspace_layout(int d, int f, int E, int k, int n_shared, int max_tokens) {
  Workspace W;
  size_t o = 0;
  const size_t tk = (size_t)max_tokens * k;
  const size_t ue = std::min<size_t>((size_t)E, tk);
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, kAlign);
    return at;
  };
  W.err = take(4);
  W.n_unique = take(4);
  W.ids = take(ue * 4);
  W.offsets = take((ue + 1) * 4);
  W.pair_token = take(tk * 4);
  W.pair_slot = take(tk * 4);
  W.pair_of = take(tk * 4);
  W.logits = take((size_t)max_tokens * E * 4);
  W.rpart = take((size_t)router_splits(d) * max_tokens * E * 4);
  const size_t rows = tk + (size_t)max_tokens * n_shared;
  W.h = take(rows * f * 4);
  W.y = take(rows * d * 4);
  W.xq = take((size_t)max_tokens * (d / kChunk) * kDigitWords * 4);
  W.xs = take((size_t)max_tokens * (d / 16) * 4);
  W.hq = take(rows * (f / kChunk) * kDigitWords * 4);
  W.hs = take(rows * (f / 16) * 4);
  W.xb = take(rows * d * 2);
  W.hb = take(rows * f * 2);
  W.mblk_max = mfma_max_entries(max_tokens, k, E, n_shared);
  W.mblk = take((size_t)W.mblk_max * 2 * 16);  // one-M-tile blocks, then the larger ones
  W.mcount = take(8);
  W.wslot = take(32 * 4);
  W.bytes = o;
  return W;
}

}  // namespace colimoe

enum { PATH_FP32 = 0, PATH_FXP = 1, PATH_MFMA = 2, PATH_I8 = 3 };

// Arithmetic path of a forward call.  AUTO: the bf16 MFMA path for
// prefill-shaped calls (on average at least 64 tokens per expert, T*k >= 64*E),
// else the fixed-point activation path when the shapes allow it (d and f at
// least 2048), else fp32 dequantisation.
static int select_path(colimoe_ctx *ctx, int T, uint32_t flags) {
  const Dims D = dims_of(ctx, T);
  if (ctx->cfg.flags & COLIMOE_CFG_INT8) {  // int8 experts: fp32 dequantisation, any T
    if (flags != COLIMOE_FWD_AUTO && flags != COLIMOE_FWD_FP32) return COLIMOE_E_SHAPE;
    return PATH_I8;
  }
  if (flags == COLIMOE_FWD_BF16_MFMA) return PATH_MFMA;
  if (flags == COLIMOE_FWD_FP32) return PATH_FP32;
  if (flags == COLIMOE_FWD_FXP) return fxp_supported(D) ? PATH_FXP : COLIMOE_E_SHAPE;
  if (flags != COLIMOE_FWD_AUTO) return COLIMOE_E_ARG;
  if ((long)T * D.k >= 64L * D.E) return PATH_MFMA;
  return fxp_supported(D) ? PATH_FXP : PATH_FP32;
}

static colimoe_union ws_union_abi(colimoe_ctx *ctx) {
  const UnionDev U = ws_union(ctx);
  colimoe_union u;
  u.n_unique = U.n_unique;
  u.ids = U.ids;
  u.offsets = U.offsets;
  u.pair_token = U.pair_token;
  u.pair_slot = U.pair_slot;
  u.pair_of = U.pair_of;
  return u;
}

// Router, top-k and (if u) union lists; `encode` also writes the fixed-point
// encoding of x into the workspace when the route runs as one kernel, and
// `shared_early` (up to 4 tokens) runs the shared expert's fixed-point
// gate/up in the top-k launch.
static int route_impl(colimoe_ctx *ctx, int32_t layer, const float *x, int32_t T, int32_t *idx, float *w,
               const colimoe_union *u, float *logits, bool encode, bool shared_early = false) {
  const Dims D = dims_of(ctx, T);
  const LayerDev L = layer_of(ctx, layer);
  float *lg = logits ? logits : (float *)(ctx->ws + ctx->wl.logits);
  hipStream_t s = ctx->stream;
  int32_t *err = (int32_t *)(ctx->ws + ctx->wl.err);
  if (D.T == 1 && !encode && !shared_early && route_one_small_supported(D)) {
    KTimer kt(ctx, K_ROUTE);
    const UnionDev U = u ? to_dev(u) : UnionDev{};
    if (launch_route_one_small(L, D, x, lg, idx, w, u ? &U : nullptr, ctx->top_p, s) != hipSuccess)
      return COLIMOE_E_HIP;
    return COLIMOE_OK;
  }
  if (D.T <= kRouteSplitMaxT) {
    {
      KTimer kt(ctx, K_ROUTE);
      uint32_t *xq = encode ? (uint32_t *)(ctx->ws + ctx->wl.xq) : nullptr;
      float *xs = encode ? (float *)(ctx->ws + ctx->wl.xs) : nullptr;
      if (launch_router_split(L, D, x, lg, xq, xs, s) != hipSuccess) return COLIMOE_E_HIP;
    }
    if (D.T == 1) {
      KTimer kt(ctx, K_TOPK);
      const UnionDev U = u ? to_dev(u) : UnionDev{};
      if (shared_early) {
        if (launch_topk_shared1(lg, D, idx, w, u ? &U : nullptr, ctx->top_p, L, (uint32_t *)(ctx->ws + ctx->wl.xq),
                                (float *)(ctx->ws + ctx->wl.xs), (uint32_t *)(ctx->ws + ctx->wl.hq),
                                (float *)(ctx->ws + ctx->wl.hs), s) != hipSuccess)
          return COLIMOE_E_HIP;
      } else if (launch_topk_union1(lg, D, idx, w, u ? &U : nullptr, ctx->top_p, s) != hipSuccess) {
        return COLIMOE_E_HIP;
      }
      return COLIMOE_OK;
    }
    if (u) {  // up to 16 tokens: top-k and the union lists in one launch
      KTimer kt(ctx, K_TOPK);
      if (shared_early) {
        if (launch_topk_union_shared(lg, D, idx, w, to_dev(u), err, ctx->top_p, L, (uint32_t *)(ctx->ws + ctx->wl.xq),
                                     (float *)(ctx->ws + ctx->wl.xs), (uint32_t *)(ctx->ws + ctx->wl.hq),
                                     (float *)(ctx->ws + ctx->wl.hs), s) != hipSuccess)
          return COLIMOE_E_HIP;
      } else if (launch_topk_union(lg, D, idx, w, to_dev(u), err, ctx->top_p, s) != hipSuccess) {
        return COLIMOE_E_HIP;
      }
      return COLIMOE_OK;
    }
  } else {
    KTimer kt(ctx, K_ROUTE);
    if (launch_router_mfma(L, D, x, (float *)(ctx->ws + ctx->wl.rpart), lg, s) != hipSuccess) return COLIMOE_E_HIP;
  }
  {
    KTimer kt(ctx, K_TOPK);
    if (launch_topk(lg, D, idx, w, ctx->top_p, s) != hipSuccess) return COLIMOE_E_HIP;
  }
  if (u) {
    KTimer kt(ctx, K_UNION);
    if (launch_union(idx, D, to_dev(u), err, s) != hipSuccess) return COLIMOE_E_HIP;
  }
  return COLIMOE_OK;
}

// Expert work and combine.  x_encoded: the workspace already holds the
// fixed-point encoding of this x (written by the route kernel); shared_done:
// also the shared expert's h encoding (written by the top-k launch).
static int forward_kernels(colimoe_ctx *ctx, int32_t layer, const float *x, int32_t T, const int32_t *idx, const float *w,
                 const colimoe_union *u, float *residual, int path, bool x_encoded, bool shared_done) {
  const Dims D = dims_of(ctx, T);
  const LayerDev L = layer_of(ctx, layer);
  hipStream_t s = ctx->stream;

  UnionDev U;
  if (u) {
    U = to_dev(u);
  } else {
    U = ws_union(ctx);
    KTimer kt(ctx, K_UNION);
    if (launch_union(idx, D, U, (int32_t *)(ctx->ws + ctx->wl.err), s) != hipSuccess) return COLIMOE_E_HIP;
  }
  float *h = (float *)(ctx->ws + ctx->wl.h);
  float *y = (float *)(ctx->ws + ctx->wl.y);
  const bool fused = (path == PATH_FP32 && (down_fusable(D) || narrow_dec_supported(D))) ||
                     (path == PATH_I8 && (i8_dec_supported(D) || i8_tok_supported(D)));
  if (path == PATH_I8) {
    KTimer kt(ctx, K_GATEUP);
    if (fused && D.T == 1) {
      if (launch_forward_i8_dec(L, D, x, U, h, w, residual, s) != hipSuccess) return COLIMOE_E_HIP;
    } else if (fused) {
      if (launch_forward_i8_tok(L, D, x, U, idx, h, w, residual, s) != hipSuccess) return COLIMOE_E_HIP;
    } else if (launch_forward_i8(L, D, x, U, h, y, s) != hipSuccess) {
      return COLIMOE_E_HIP;
    }
  } else if (path == PATH_MFMA) {
    int4 *list = (int4 *)(ctx->ws + ctx->wl.mblk);
    int32_t *mcount = (int32_t *)(ctx->ws + ctx->wl.mcount);
    uint16_t *xb = (uint16_t *)(ctx->ws + ctx->wl.xb);
    uint16_t *hb = (uint16_t *)(ctx->ws + ctx->wl.hb);
    const int me = mfma_max_entries(T, D.k, D.E, D.n_shared);
    {
      KTimer kt(ctx, K_ENCODE);
      if (launch_mblocks(D, U, list, mcount, me, s) != hipSuccess) return COLIMOE_E_HIP;
      if (launch_gather_bf16(x, D, xb, s) != hipSuccess) return COLIMOE_E_HIP;
    }
    {
      KTimer kt(ctx, K_GATEUP);
      if (launch_gateup_mfma(L, D, xb, U, list, mcount, me, hb, s) != hipSuccess) return COLIMOE_E_HIP;
    }
    {
      KTimer kt(ctx, K_DOWN);
      if (launch_down_mfma(L, D, hb, list, mcount, me, y, s) != hipSuccess) return COLIMOE_E_HIP;
    }
  } else if (path == PATH_FXP) {
    uint32_t *xq = (uint32_t *)(ctx->ws + ctx->wl.xq);
    float *xs = (float *)(ctx->ws + ctx->wl.xs);
    uint32_t *hq = (uint32_t *)(ctx->ws + ctx->wl.hq);
    float *hs = (float *)(ctx->ws + ctx->wl.hs);
    float *wslot = (float *)(ctx->ws + ctx->wl.wslot);
    if (!x_encoded) {
      KTimer kt(ctx, K_ENCODE);
      if (launch_xquant(x, T, D.d, xq, xs, s) != hipSuccess) return COLIMOE_E_HIP;
    }
    {
      KTimer kt(ctx, K_GATEUP);
      if (launch_gateup_tok(L, D, U, idx, w, xq, xs, hq, hs, wslot, shared_done, s) != hipSuccess) return COLIMOE_E_HIP;
    }
    if (down_dec_supported(D)) {
      KTimer kt(ctx, K_DOWN);
      if (launch_down_dec(L, D, hq, hs, U, wslot, residual, s) != hipSuccess) return COLIMOE_E_HIP;
      return COLIMOE_OK;  // combine done in the kernel
    }
    if (down_dec_tok_supported(D)) {
      KTimer kt(ctx, K_DOWN);
      if (launch_down_dec_tok(L, D, hq, hs, U, idx, w, residual, s) != hipSuccess) return COLIMOE_E_HIP;
      return COLIMOE_OK;  // combine done in the kernel
    }
    {
      KTimer kt(ctx, K_DOWN);
      if (launch_down_tok(L, D, U, hq, hs, y, s) != hipSuccess) return COLIMOE_E_HIP;
    }
  } else if (fused && f32_dec_supported(D)) {
    float *hsum = (float *)(ctx->ws + ctx->wl.hs);
    {
      KTimer kt(ctx, K_GATEUP);
      if (launch_gateup_f32_dec(L, D, x, U, h, hsum, s) != hipSuccess) return COLIMOE_E_HIP;
    }
    {
      KTimer kt(ctx, K_DOWN);
      if (launch_down_f32_dec(L, D, h, hsum, U, w, residual, s) != hipSuccess) return COLIMOE_E_HIP;
    }
  } else if (fused && f32_dec_tok_supported(D)) {
    KTimer kt(ctx, K_GATEUP);  // gate/up and down with the combine (two launches)
    if (launch_f32_dec_tok(L, D, x, U, idx, w, h, (float *)(ctx->ws + ctx->wl.hs), residual, s) != hipSuccess)
      return COLIMOE_E_HIP;
  } else {
    {
      KTimer kt(ctx, K_GATEUP);
      if (launch_gateup(L, D, x, U, h, s) != hipSuccess) return COLIMOE_E_HIP;
    }
    {
      KTimer kt(ctx, K_DOWN);
      if (launch_down(L, D, h, U, y, w, residual, fused, s) != hipSuccess) return COLIMOE_E_HIP;
    }
  }
  if (!fused) {
    KTimer kt(ctx, K_COMBINE);
    if (launch_combine(D, w, U, y, residual, s) != hipSuccess) return COLIMOE_E_HIP;
  }
  return COLIMOE_OK;
}

// On a host-resident layer the call's experts are first made present in the
// HBM cache; then, with prefetch on, the next layer's router starts on x (one
// layer ahead) beside this layer's kernels, and its predicted experts start
// moving into the cache once the prediction is in.
static int forward_impl(colimoe_ctx *ctx, int32_t layer, const float *x, int32_t T, const int32_t *idx, const float *w,
                        const colimoe_union *u, float *residual, int path, bool x_encoded, bool shared_done = false) {
  int predicting = 0;
  if (ctx->host_store[layer]) {
    const int rc = cache_ensure_resident(ctx, layer, idx, T);
    if (rc) return rc;
    predicting = cache_predict_start(ctx, layer, x, T);
    if (predicting < 0) return predicting;
  }
  const int rc = forward_kernels(ctx, layer, x, T, idx, w, u, residual, path, x_encoded, shared_done);
  const int rp = predicting ? cache_prefetch_issue(ctx, layer, T) : COLIMOE_OK;
  return rc ? rc : rp;
}

extern "C" {

const char *colimoe_status_str(int s) {
  switch (s) {
    case COLIMOE_OK: return "ok";
    case COLIMOE_E_ARG: return "invalid argument (null or misaligned pointer, bad flag, index or routing)";
    case COLIMOE_E_SHAPE: return "invalid shape (config, layer index or token count)";
    case COLIMOE_E_NOT_LOADED: return "layer not loaded";
    case COLIMOE_E_WORKSPACE: return "workspace missing or too small";
    case COLIMOE_E_HIP: return "HIP runtime error";
    case COLIMOE_E_STATE: return "call out of order";
    default: return "unknown status";
  }
}

size_t colimoe_expert_bytes(const colimoe_config *cfg) {
  if (!cfg_ok(cfg)) return 0;
  return cfg_expert_bytes(cfg);
}

size_t colimoe_layer_bytes(const colimoe_config *cfg) {
  if (!cfg_ok(cfg)) return 0;
  return router_bytes(cfg) + (size_t)(cfg->n_experts + cfg->n_shared) * cfg_expert_bytes(cfg);
}

size_t colimoe_workspace_bytes(const colimoe_config *cfg) {
  if (!cfg_ok(cfg)) return 0;
  return workspace_layout(cfg->d, cfg->f, cfg->n_experts, cfg->top_k, cfg->n_shared, cfg->max_tokens).bytes;
}

int colimoe_create(const colimoe_config *cfg, void *hip_stream, colimoe_ctx **out) {
  if (!out) return COLIMOE_E_ARG;
  *out = nullptr;
  if (!cfg) return COLIMOE_E_ARG;
  if (!cfg_ok(cfg)) return COLIMOE_E_SHAPE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return COLIMOE_E_HIP;
  colimoe_ctx *c = new colimoe_ctx();
  c->cfg = *cfg;
  c->stream = (hipStream_t)hip_stream;
  c->device = dev;
  c->layers.assign(cfg->n_layers, LayerDev{nullptr, nullptr, nullptr, 0, nullptr});
  c->loaded.assign(cfg->n_layers, 0);
  c->host_store.assign(cfg->n_layers, nullptr);
  c->ws = nullptr;
  c->ws_bytes = 0;
  c->static_used = false;
  // The static scratch's address on this device, looked up once per device
  // while it is current.  A failure here only disables
  // colimoe_route_forward_static (it then returns E_HIP).
  (void)static_scratch_init(dev);
  c->top_p = 1.0f;
  c->wl = workspace_layout(cfg->d, cfg->f, cfg->n_experts, cfg->top_k, cfg->n_shared, cfg->max_tokens);
  c->el = expert_layout(cfg->d, cfg->f);
  c->el.bytes = cfg_expert_bytes(cfg);  // the int8 container keeps the canonical layout
  c->staging[0] = c->staging[1] = nullptr;
  c->staging_bytes = 0;
  c->timing = false;
  c->ev_used = 0;
  for (int i = 0; i < 16; ++i) {
    c->tot_ms[i] = 0.0;
    c->cnt[i] = 0;
  }
  *out = c;
  return COLIMOE_OK;
}

void colimoe_destroy(colimoe_ctx *ctx) {
  if (!ctx) return;
  cache_release(ctx);
  for (int i = 0; i < 2; ++i)
    if (ctx->staging[i]) (void)hipHostFree(ctx->staging[i]);
  for (hipEvent_t e : ctx->ev_pool) (void)hipEventDestroy(e);
  delete ctx;
}

int colimoe_set_expert_top_p(colimoe_ctx *ctx, float p) {
  if (!ctx || !(p > 0.0f && p <= 1.0f)) return COLIMOE_E_ARG;
  ctx->top_p = p;
  return COLIMOE_OK;
}

int colimoe_set_stream(colimoe_ctx *ctx, void *hip_stream) {
  if (!ctx) return COLIMOE_E_ARG;
  ctx->stream = (hipStream_t)hip_stream;
  return COLIMOE_OK;
}

int colimoe_set_workspace(colimoe_ctx *ctx, void *dev, size_t bytes) {
  if (!ctx || !dev || !aligned(dev, kAlign)) return COLIMOE_E_ARG;
  if (bytes < ctx->wl.bytes) return COLIMOE_E_WORKSPACE;
  ctx->ws = (uint8_t *)dev;
  ctx->ws_bytes = bytes;
  return hip_status(hipMemsetAsync(ctx->ws + ctx->wl.err, 0, 4, ctx->stream));
}

int colimoe_load_experts(colimoe_ctx *ctx, int32_t layer, const colimoe_layer_src *src, void *dev_dst,
                         size_t dev_bytes) {
  if (!ctx || !src || !dev_dst || !src->router || !src->experts) return COLIMOE_E_ARG;
  const colimoe_config *c = &ctx->cfg;
  if (layer < 0 || layer >= c->n_layers) return COLIMOE_E_SHAPE;
  if ((c->n_shared == 1) != (src->shared != nullptr)) return COLIMOE_E_ARG;
  if (!aligned(dev_dst, kAlign)) return COLIMOE_E_ARG;
  if (dev_bytes < colimoe_layer_bytes(c)) return COLIMOE_E_SHAPE;
  const size_t be = ctx->el.bytes;
  uint8_t *dst = (uint8_t *)dev_dst;
  hipStream_t s = ctx->stream;
  const size_t rb = (size_t)c->n_experts * c->d * 4;
  float *router = (float *)dst;
  float *bias = (float *)(dst + align_up(rb, kAlign));
  uint8_t *experts = dst + router_bytes(c);
  ctx->loaded[layer] = 0;
  cache_drop_layer(ctx, layer);
  if (hipMemcpyAsync(router, src->router, rb, hipMemcpyHostToDevice, s) != hipSuccess) return COLIMOE_E_HIP;
  if (src->bias) {
    if (hipMemcpyAsync(bias, src->bias, (size_t)c->n_experts * 4, hipMemcpyHostToDevice, s) != hipSuccess)
      return COLIMOE_E_HIP;
  } else if (hipMemsetAsync(bias, 0, (size_t)c->n_experts * 4, s) != hipSuccess) {
    return COLIMOE_E_HIP;
  }
  // Repack batches of experts into pinned staging buffers, double-buffered
  // against the host-to-device copies.
  const int total = c->n_experts + c->n_shared;
  const int per = (int)std::max<size_t>(1, std::min<size_t>((size_t)total, ((size_t)256 << 20) / be));
  if (ctx->staging_bytes < (size_t)per * be) {
    for (int i = 0; i < 2; ++i) {
      if (ctx->staging[i]) (void)hipHostFree(ctx->staging[i]);
      ctx->staging[i] = nullptr;
    }
    ctx->staging_bytes = 0;
    for (int i = 0; i < 2; ++i)
      if (hipHostMalloc((void **)&ctx->staging[i], (size_t)per * be, hipHostMallocDefault) != hipSuccess)
        return COLIMOE_E_HIP;
    ctx->staging_bytes = (size_t)per * be;
  }
  hipEvent_t done[2];
  if (hipEventCreateWithFlags(&done[0], hipEventDisableTiming) != hipSuccess) return COLIMOE_E_HIP;
  if (hipEventCreateWithFlags(&done[1], hipEventDisableTiming) != hipSuccess) return COLIMOE_E_HIP;
  bool used[2] = {false, false};
  int rc = COLIMOE_OK;
  std::vector<const uint8_t *> srcs(per);
  for (int e0 = 0, b = 0; e0 < total && rc == COLIMOE_OK; e0 += per, b ^= 1) {
    const int n = std::min(per, total - e0);
    if (used[b] && hipEventSynchronize(done[b]) != hipSuccess) {
      rc = COLIMOE_E_HIP;
      break;
    }
    for (int i = 0; i < n; ++i) {
      const int e = e0 + i;
      srcs[i] = e < c->n_experts ? src->experts + (size_t)e * be : src->shared;
    }
    if (c->flags & COLIMOE_CFG_INT8)
      copy_many(srcs.data(), ctx->staging[b], n, be);
    else
      repack_many(srcs.data(), ctx->staging[b], n, be, c->d, c->f);
    if (hipMemcpyAsync(experts + (size_t)e0 * be, ctx->staging[b], (size_t)n * be, hipMemcpyHostToDevice, s) !=
            hipSuccess ||
        hipEventRecord(done[b], s) != hipSuccess)
      rc = COLIMOE_E_HIP;
    used[b] = true;
  }
  if (hipStreamSynchronize(s) != hipSuccess) rc = COLIMOE_E_HIP;
  (void)hipEventDestroy(done[0]);
  (void)hipEventDestroy(done[1]);
  if (rc != COLIMOE_OK) return rc;
  ctx->layers[layer] = LayerDev{router, bias, experts, be, nullptr};
  ctx->loaded[layer] = 1;
  return COLIMOE_OK;
}

int colimoe_route(colimoe_ctx *ctx, int32_t layer, const float *x, int32_t T, int32_t *idx, float *w,
                  const colimoe_union *u, float *logits) {
  int rc = check_call(ctx, layer, T);
  if (rc) return rc;
  if (T == 0) return COLIMOE_OK;  // nothing to read or write; pointers may be NULL
  if (!x || !idx || !w || !aligned(x, 16) || !aligned(idx, 4) || !aligned(w, 4)) return COLIMOE_E_ARG;
  if (logits && !aligned(logits, 4)) return COLIMOE_E_ARG;
  if (u && !union_ok(u)) return COLIMOE_E_ARG;
  return route_impl(ctx, layer, x, T, idx, w, u, logits, false);
}

int colimoe_union_build(colimoe_ctx *ctx, const int32_t *idx, int32_t T, const colimoe_union *u) {
  if (!ctx) return COLIMOE_E_ARG;
  if (T < 0 || T > ctx->cfg.max_tokens) return COLIMOE_E_SHAPE;
  if (!ctx->ws) return COLIMOE_E_WORKSPACE;
  if (T == 0) return COLIMOE_OK;
  if (!idx || !aligned(idx, 4) || !union_ok(u)) return COLIMOE_E_ARG;
  const Dims D = dims_of(ctx, T);
  return hip_status(launch_union(idx, D, to_dev(u), (int32_t *)(ctx->ws + ctx->wl.err), ctx->stream));
}

int colimoe_forward(colimoe_ctx *ctx, int32_t layer, const float *x, int32_t T, const int32_t *idx, const float *w,
                    const colimoe_union *u, float *residual, uint32_t flags) {
  int rc = check_call(ctx, layer, T);
  if (rc) return rc;
  if (flags > COLIMOE_FWD_FXP) return COLIMOE_E_ARG;
  if (T == 0) return COLIMOE_OK;  // nothing to read or write; pointers may be NULL
  if (!x || !idx || !w || !residual || !aligned(x, 16) || !aligned(idx, 4) || !aligned(w, 4) ||
      !aligned(residual, 16))
    return COLIMOE_E_ARG;
  if (u && !union_ok(u)) return COLIMOE_E_ARG;
  int path = select_path(ctx, T, flags);
  if (path < 0) return path;
  return forward_impl(ctx, layer, x, T, idx, w, u, residual, path, false);
}

int colimoe_route_forward(colimoe_ctx *ctx, int32_t layer, const float *x, int32_t T, int32_t *idx, float *w,
                          const colimoe_union *u, float *residual, uint32_t flags) {
  int rc = check_call(ctx, layer, T);
  if (rc) return rc;
  if (flags > COLIMOE_FWD_FXP) return COLIMOE_E_ARG;
  if (T == 0) return COLIMOE_OK;
  if (!x || !idx || !w || !residual || !aligned(x, 16) || !aligned(idx, 4) || !aligned(w, 4) ||
      !aligned(residual, 16))
    return COLIMOE_E_ARG;
  if (u && !union_ok(u)) return COLIMOE_E_ARG;
  const int path = select_path(ctx, T, flags);
  if (path < 0) return path;
  const colimoe_union uw = ws_union_abi(ctx);
  const colimoe_union *uu = u ? u : &uw;
  const bool encode = path == PATH_FXP;
  const Dims D = dims_of(ctx, T);
  // up to 4 tokens on an HBM-resident layer: the shared expert's gate/up
  // rides in the top-k launch
  const bool early =
      encode && !ctx->host_store[layer] && (shared_early_supported(D) || shared_early_multi_supported(D));
  rc = route_impl(ctx, layer, x, T, idx, w, uu, nullptr, encode, early);
  if (rc) return rc;
  return forward_impl(ctx, layer, x, T, idx, w, uu, residual, path, encode && T <= kRouteSplitMaxT, early);
}

int colimoe_route_forward_static(colimoe_ctx *ctx, int32_t layer, const float *x, int32_t T, int32_t *idx,
                                 float *w, const colimoe_union *u, float *residual, uint32_t flags) {
  if (!ctx) return COLIMOE_E_ARG;
  if (layer < 0 || layer >= ctx->cfg.n_layers) return COLIMOE_E_SHAPE;
  if (T < 0 || T > ctx->cfg.max_tokens) return COLIMOE_E_SHAPE;
  if (!ctx->loaded[layer]) return COLIMOE_E_NOT_LOADED;
  if (flags > COLIMOE_FWD_FXP) return COLIMOE_E_ARG;
  if (T == 0) return COLIMOE_OK;
  if (!x || !idx || !w || !residual || !aligned(x, 16) || !aligned(idx, 4) || !aligned(w, 4) ||
      !aligned(residual, 16))
    return COLIMOE_E_ARG;
  if (u && !union_ok(u)) return COLIMOE_E_ARG;
  const int path = select_path(ctx, T, flags);
  if (path < 0) return path;
  // the workspace this call needs, laid out for its own T
  const Workspace wl =
      workspace_layout(ctx->cfg.d, ctx->cfg.f, ctx->cfg.n_experts, ctx->cfg.top_k, ctx->cfg.n_shared, T);
  if (wl.bytes > kStaticScratchBytes) return COLIMOE_E_WORKSPACE;
  uint8_t *scr = static_scratch(ctx->device);
  if (!scr) return COLIMOE_E_HIP;  // the address lookup at colimoe_create failed
  // The same launches as colimoe_route_forward, with the scratch standing in
  // for the context's workspace; timing is off (its events are created on
  // demand), and everything is put back before returning.
  uint8_t *const ws = ctx->ws;
  const size_t ws_bytes = ctx->ws_bytes;
  const Workspace saved = ctx->wl;
  const bool timing = ctx->timing;
  ctx->ws = scr;
  ctx->ws_bytes = kStaticScratchBytes;
  ctx->wl = wl;
  ctx->timing = false;
  ctx->static_used = true;
  // the error word must start at zero; the scratch keeps the last call's contents
  int rc = hip_status(launch_zero_words((uint32_t *)(scr + wl.err), 1, ctx->stream));
  if (!rc) rc = colimoe_route_forward(ctx, layer, x, T, idx, w, u, residual, flags);
  ctx->ws = ws;
  ctx->ws_bytes = ws_bytes;
  ctx->wl = saved;
  ctx->timing = timing;
  return rc;
}

int colimoe_rmsnorm_route_forward(colimoe_ctx *ctx, int32_t layer, float *r, int32_t T, float eps, float *x_out,
                                  int32_t *idx, float *w, const colimoe_union *u, uint32_t flags) {
  int rc = check_call(ctx, layer, T);
  if (rc) return rc;
  if (flags > COLIMOE_FWD_FXP) return COLIMOE_E_ARG;
  if (!(eps >= 0.0f)) return COLIMOE_E_ARG;
  if (T == 0) return COLIMOE_OK;
  if (!r || !x_out || !idx || !w || !aligned(r, 16) || !aligned(x_out, 16) || !aligned(idx, 4) || !aligned(w, 4))
    return COLIMOE_E_ARG;
  if (u && !union_ok(u)) return COLIMOE_E_ARG;
  const int path = select_path(ctx, T, flags);
  if (path < 0) return path;
  const Dims D = dims_of(ctx, T);
  if (T != 1 || path != PATH_FXP) {  // the two calls it stands for
    {
      KTimer kt(ctx, K_RMSNORM);
      rc = hip_status(launch_rmsnorm(r, T, ctx->cfg.d, eps, x_out, ctx->stream));
    }
    if (rc) return rc;
    return colimoe_route_forward(ctx, layer, x_out, T, idx, w, u, r, flags);
  }
  const colimoe_union uw = ws_union_abi(ctx);
  const colimoe_union *uu = u ? u : &uw;
  const LayerDev L = layer_of(ctx, layer);
  {
    KTimer kt(ctx, K_ROUTE);
    if (launch_router_norm(L, D, r, eps, x_out, (float *)(ctx->ws + ctx->wl.logits), (uint32_t *)(ctx->ws + ctx->wl.xq),
                           (float *)(ctx->ws + ctx->wl.xs), ctx->stream) != hipSuccess)
      return COLIMOE_E_HIP;
  }
  const bool early = !ctx->host_store[layer] && shared_early_supported(D);
  {
    KTimer kt(ctx, K_TOPK);
    const UnionDev U = to_dev(uu);
    float *lg = (float *)(ctx->ws + ctx->wl.logits);
    if (early) {
      if (launch_topk_shared1(lg, D, idx, w, &U, ctx->top_p, L, (uint32_t *)(ctx->ws + ctx->wl.xq),
                              (float *)(ctx->ws + ctx->wl.xs), (uint32_t *)(ctx->ws + ctx->wl.hq),
                              (float *)(ctx->ws + ctx->wl.hs), ctx->stream) != hipSuccess)
        return COLIMOE_E_HIP;
    } else if (launch_topk_union1(lg, D, idx, w, &U, ctx->top_p, ctx->stream) != hipSuccess) {
      return COLIMOE_E_HIP;
    }
  }
  return forward_impl(ctx, layer, x_out, T, idx, w, uu, r, path, true, early);
}

int colimoe_rmsnorm(colimoe_ctx *ctx, const float *r, int32_t T, float eps, float *x_out) {
  if (!ctx) return COLIMOE_E_ARG;
  if (T < 0 || T > ctx->cfg.max_tokens) return COLIMOE_E_SHAPE;
  if (!(eps >= 0.0f)) return COLIMOE_E_ARG;
  if (T == 0) return COLIMOE_OK;
  if (!r || !x_out || !aligned(r, 16) || !aligned(x_out, 16)) return COLIMOE_E_ARG;
  KTimer kt(ctx, K_RMSNORM);
  return hip_status(launch_rmsnorm(r, T, ctx->cfg.d, eps, x_out, ctx->stream));
}

int colimoe_debug_expert(colimoe_ctx *ctx, int32_t layer, int32_t e, const float *x, float *g, float *u, float *h,
                         float *y) {
  int rc = check_call(ctx, layer, 1);
  if (rc) return rc;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 4)) return COLIMOE_E_ARG;
  if ((g == nullptr) != (u == nullptr)) return COLIMOE_E_ARG;
  if (e < -1 || e >= ctx->cfg.n_experts) return COLIMOE_E_ARG;
  if (e == -1 && ctx->cfg.n_shared == 0) return COLIMOE_E_ARG;
  if (ctx->host_store[layer]) return COLIMOE_E_STATE;  // experts of a host-resident layer are not all in HBM
  if (ctx->cfg.flags & COLIMOE_CFG_INT8) return COLIMOE_E_SHAPE;  // the stage-by-stage path reads int4
  const int slot = e < 0 ? ctx->cfg.n_experts : e;
  // a one-slot union in the workspace: expert `slot`, one pair (token 0)
  Dims D = dims_of(ctx, 1);
  D.k = 1;
  D.n_shared = 0;
  D.E = ctx->cfg.n_experts + 1;  // admits the shared expert's storage index
  UnionDev U = ws_union(ctx);
  const int32_t host[7] = {1, slot, 0, 1, 0, 0, 0};
  hipStream_t s = ctx->stream;
  if (hipMemcpyAsync(U.n_unique, &host[0], 4, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(U.ids, &host[1], 4, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(U.offsets, &host[2], 8, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(U.pair_token, &host[4], 4, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(U.pair_slot, &host[5], 4, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(U.pair_of, &host[6], 4, hipMemcpyHostToDevice, s) != hipSuccess)
    return COLIMOE_E_HIP;
  float *hh = h ? h : (float *)(ctx->ws + ctx->wl.h);
  const LayerDev L = layer_of(ctx, layer);
  if (launch_debug_gateup(L, D, x, U, hh, g, u, s) != hipSuccess) return COLIMOE_E_HIP;
  if (launch_down(L, D, hh, U, y, nullptr, nullptr, false, s) != hipSuccess) return COLIMOE_E_HIP;
  return hip_status(hipStreamSynchronize(s));  // keeps `host` alive for the copies
}

int colimoe_timing_enable(colimoe_ctx *ctx, int enable) {
  if (!ctx) return COLIMOE_E_ARG;
  ctx->timing = enable != 0;
  return COLIMOE_OK;
}

int colimoe_timing_read(colimoe_ctx *ctx, const char *name, double *total_ms, int64_t *count, int reset) {
  if (!ctx || !name || !total_ms || !count) return COLIMOE_E_ARG;
  int kid = -1;
  for (int i = 0; i < K_COUNT; ++i)
    if (strcmp(name, kKernelNames[i]) == 0) kid = i;
  if (kid < 0) return COLIMOE_E_ARG;
  int rc = drain_timing(ctx);
  if (rc) return rc;
  *total_ms = ctx->tot_ms[kid];
  *count = ctx->cnt[kid];
  if (reset)
    for (int i = 0; i < 16; ++i) {
      ctx->tot_ms[i] = 0.0;
      ctx->cnt[i] = 0;
    }
  return COLIMOE_OK;
}

int colimoe_sync(colimoe_ctx *ctx) {
  if (!ctx) return COLIMOE_E_ARG;
  if (hipStreamSynchronize(ctx->stream) != hipSuccess) return COLIMOE_E_HIP;
  // the error word of the workspace, and of the static scratch once used
  // (the error word sits at offset 0 of every workspace layout)
  uint8_t *words[2] = {ctx->ws ? ctx->ws + ctx->wl.err : nullptr,
                       ctx->static_used ? static_scratch(ctx->device) : nullptr};
  int rc = COLIMOE_OK;
  for (uint8_t *p : words) {
    if (!p) continue;
    int32_t err = 0;
    if (hipMemcpy(&err, p, 4, hipMemcpyDeviceToHost) != hipSuccess) return COLIMOE_E_HIP;
    if (err) {
      if (hipMemset(p, 0, 4) != hipSuccess) return COLIMOE_E_HIP;
      rc = COLIMOE_E_ARG;
    }
  }
  return rc;
}

}  // extern "C"
