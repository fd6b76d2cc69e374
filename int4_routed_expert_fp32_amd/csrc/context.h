// context.h - the library's host-side context (private to host.cpp and
// cache.cpp; not part of the public ABI) and the helpers the two share.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/colimoe.h"
#include "internal.h"

namespace colimoe {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline int hip_status(hipError_t e) { return e == hipSuccess ? COLIMOE_OK : COLIMOE_E_HIP; }

// Tiered placement (cache.cpp): routed experts of host-resident layers live
// in pinned host memory (device layout) and are brought into an HBM cache of
// expert slots on demand.  The slots are split evenly among the context's
// layers; layer l owns slots [l * per_layer, (l + 1) * per_layer), with its
// own least-recently-used order, its shared expert fixed in its first slot,
// and its learned (pinned) experts.
struct ExpertCache {
  uint8_t *slots = nullptr;       // device: n_slots * expert bytes
  int32_t *dev_maps = nullptr;    // device: [n_layers][E + 1] slot of each expert
  float *pred_logits = nullptr;   // device: [16][E] logits of a prediction
  int32_t *pred_idx = nullptr;    // device: [16][k] its top-k
  float *pred_w = nullptr;        // device: [16][k] (unused weights of that top-k)
  int32_t *stage = nullptr;       // pinned host: the maps as uploaded
  int32_t *idx_host = nullptr;    // pinned host: a call's routing
  int32_t *pred_host = nullptr;   // pinned host: a prediction's routing
  int n_slots = 0, per_layer = 0;
  std::vector<int32_t> slot_of;   // [n_layers][E + 1]: global slot or -1
  std::vector<int32_t> tag;       // per slot: expert id (E: shared) held, or -1
  std::vector<uint64_t> used;     // per slot: stamp of the last use
  std::vector<char> fixed;        // per slot: 1 shared expert, 2 pinned expert (neither evicted)
  std::vector<char> fresh;        // per slot: brought in by a prediction, not yet needed by a call
  std::vector<uint32_t> uses;     // [n_layers][E]: tokens routed to each expert (usage histogram)
  std::vector<int64_t> tokens;    // per layer: tokens served since the last automatic repin
  std::vector<std::vector<int32_t>> pred;  // per layer: experts the last prediction named (sorted)
  std::vector<char> pending;       // per slot: a prefetch copy into it may still be running
  std::vector<hipEvent_t> ev_slot;  // per slot: end of the latest prefetch copy into it
  hipStream_t copy = nullptr, side = nullptr;  // prefetch copies; the prediction router
  int prefetch = 0;               // experts of each predicted token to prefetch (0: no prediction)
  int repin_every = 0, repin_n = 0;
  uint64_t stamp = 0;
  int64_t hits = 0, misses = 0, predicted = 0, predicted_hits = 0, prefetched = 0, prefetched_used = 0;
};

}  // namespace colimoe

struct colimoe_ctx {
  colimoe_config cfg;
  hipStream_t stream;
  int device;
  std::vector<colimoe::LayerDev> layers;
  std::vector<char> loaded;
  std::vector<uint8_t *> host_store;  // per layer: E * expert bytes of pinned host memory, or null
  colimoe::ExpertCache cache;
  uint8_t *ws;
  size_t ws_bytes;
  bool static_used;  // colimoe_route_forward_static has run on this context
  float top_p;       // adaptive expert top-p of one-token routing (1: off)
  colimoe::Workspace wl;
  colimoe::ExpertLayout el;
  uint8_t *staging[2];  // pinned host buffers for the loader
  size_t staging_bytes;
  // kernel timing
  bool timing;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used;
  struct Rec {
    int kid;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  double tot_ms[16];
  long long cnt[16];
};

namespace colimoe {

// host.cpp
bool cfg_ok(const colimoe_config *c);
size_t cfg_expert_bytes(const colimoe_config *c);
size_t router_bytes(const colimoe_config *c);
Dims dims_of(const colimoe_ctx *ctx, int T);
void repack_expert(const uint8_t *src, uint8_t *dst, int d, int f);
void copy_many(const uint8_t *const *srcs, uint8_t *dst, int n, size_t be);
void repack_many(const uint8_t *const *srcs, uint8_t *dst, int n, size_t be, int d, int f);

// cache.cpp
// Makes every expert of routing idx [T][k] (device) of host-resident layer
// `layer` present in its partition before the layer's kernels run; counts
// usage and hits; runs an automatic repin when one is due.  Synchronises the
// stream (it reads the routing on the host).
int cache_ensure_resident(colimoe_ctx *ctx, int layer, const int32_t *idx, int T);
// With prefetch on and layer + 1 host-resident, for calls of up to 16
// tokens: starts predicting layer + 1's experts from this call's input x
// [T][d] (its router and top-k on the side stream; the stream was
// synchronised by cache_ensure_resident, so x is ready).  Returns 1 if a
// prediction was started, 0 if none, or an error.
int cache_predict_start(colimoe_ctx *ctx, int layer, const float *x, int T);
// Waits for that prediction (the host only) and starts copying the predicted
// experts absent from layer + 1's partition on the copy stream.
int cache_prefetch_issue(colimoe_ctx *ctx, int layer, int T);
// Forgets a layer's partition and frees its host store.
void cache_drop_layer(colimoe_ctx *ctx, int layer);
// Frees everything the cache holds (pinned buffers, streams, events).
void cache_release(colimoe_ctx *ctx);

}  // namespace colimoe
