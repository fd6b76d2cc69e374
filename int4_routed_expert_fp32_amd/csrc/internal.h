// internal.h - device data layout and kernel launchers shared by host.cpp and
// kernels.hip.  Not part of the public ABI (include/colimoe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace colimoe {

constexpr int kGroup = 64;   // int4 elements per fp16 scale
constexpr int kChunk = 32;   // elements one lane handles per 16-byte load
constexpr int kTileRows = 8; // rows of one tile (one wave reduces 8 rows at once)

// ---------------------------------------------------------------------------
// Device layout of one expert (same byte count as the canonical blob).
//
//   gu_nib  [2f rows][d/2 B]  gate and up rows interleaved by tiles of 8:
//           device row 8i+r is gate row 4i+r (r < 4) or up row 4i+r-4 (r >= 4)
//   gu_sc   [f/4 tiles][d/64 groups][8 rows] fp16
//   dn_nib  [d rows][f/2 B]   natural row order
//   dn_sc   [d/8 tiles][f/64 groups][8 rows] fp16
//
// Nibbles are stored offset-binary (n + 8, i.e. the canonical byte XOR 0x88)
// so a byte-to-float conversion yields n + 8 directly; the kernels fold the
// -8 into each chunk's starting value.  A 16-byte load of scales gives the 8
// rows of a tile their scale for one 64-wide group.
// ---------------------------------------------------------------------------
struct ExpertLayout {
  size_t gu_nib, gu_sc, dn_nib, dn_sc, bytes;
};

__host__ __device__ inline ExpertLayout expert_layout(int d, int f) {
  ExpertLayout L;
  size_t w = (size_t)d * (size_t)f;
  L.gu_nib = 0;
  L.gu_sc = w;              // 2f * d/2
  L.dn_nib = w + w / 16;    // + 2f * d/64 * 2
  L.dn_sc = L.dn_nib + w / 2;
  L.bytes = L.dn_sc + w / 32;
  return L;
}

// One loaded layer in device memory: router [E][d] fp32, bias [E] fp32, then
// E routed experts followed by the shared expert (if any), each L.bytes.
struct LayerDev {
  const float *router;
  const float *bias;
  const uint8_t *experts;
  size_t expert_stride;
};

struct Dims {
  int d, f, E, k, T, n_shared;
};

struct UnionDev {
  int32_t *n_unique, *ids, *offsets, *pair_token, *pair_slot, *pair_of;
};

// Workspace carve-up (all offsets 256-byte aligned).
struct Workspace {
  size_t err;  // int32 error word set by kernels that reject a routing
  size_t n_unique, ids, offsets, pair_token, pair_slot, pair_of;  // union lists
  size_t logits;  // [Tmax][E] fp32
  size_t h;       // [(Tmax*k + Tmax*n_shared)][f] fp32
  size_t y;       // [(Tmax*k + Tmax*n_shared)][d] fp32
  size_t bytes;
};

Workspace workspace_layout(int d, int f, int E, int k, int n_shared, int max_tokens);

// Kernel launchers (kernels.hip).  All enqueue on `s`, return hipError_t.
hipError_t launch_router(const LayerDev &L, const Dims &D, const float *x, float *logits, hipStream_t s);
hipError_t launch_topk(const float *logits, const Dims &D, int32_t *idx, float *w, hipStream_t s);
hipError_t launch_union(const int32_t *idx, const Dims &D, const UnionDev &U, int32_t *err, hipStream_t s);
hipError_t launch_gateup(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h,
                         hipStream_t s);
hipError_t launch_down(const LayerDev &L, const Dims &D, const float *h, const UnionDev &U, float *y,
                       hipStream_t s);
hipError_t launch_combine(const Dims &D, const int32_t *idx, const float *w, const UnionDev &U, const float *y,
                          float *residual, hipStream_t s);
hipError_t launch_rmsnorm(const float *r, int T, int d, float eps, float *x, hipStream_t s);
hipError_t launch_debug_gateup(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h,
                               float *g, float *u, hipStream_t s);

}  // namespace colimoe
