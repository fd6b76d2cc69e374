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
//   gu_nib  gate and up rows interleaved by tiles of 8: tile i holds gate rows
//           4i..4i+3 (tile rows 0-3) and up rows 4i..4i+3 (tile rows 4-7)
//   gu_sc   [f/4 tiles][d/64 groups][8 rows] fp16
//   dn_nib  down rows in natural order, tiles of 8
//   dn_sc   [d/8 tiles][f/64 groups][8 rows] fp16
//
// Nibble bytes of a tile (8 rows of K/2 bytes) are stored step-major: step j
// covers 32-column chunks 64j..64j+63 of all 8 rows, row after row, so the
// 8 rows x 1 KB one wave reads for a step are contiguous (rows shorter than
// 64 chunks are simply row-major within the tile).
// Nibbles keep the canonical two's-complement encoding.  A 16-byte load of
// scales gives the 8 rows of a tile their scale for one 64-wide group.
// ---------------------------------------------------------------------------

// Byte offset of chunk c (32 columns, 16 bytes) of row r of tile `tile` in a
// matrix whose rows have K columns.
__host__ __device__ inline size_t chunk_offset(int tile, int K, int c, int r) {
  const int C = K / kChunk;
  const int j = c >> 6, cl = c & 63;
  const int width = (C - 64 * j) < 64 ? (C - 64 * j) : 64;
  return (size_t)tile * kTileRows * (size_t)(K / 2) + (size_t)j * (kTileRows * 64 * 16) + (size_t)r * width * 16 +
         (size_t)cl * 16;
}

constexpr int kDigitWords = 24;               // fixed-point activations: words per 32-column chunk
constexpr int kRouteSplitMaxT = 16;           // router with K split over waves up to this many tokens
constexpr size_t kFusedLdsMax = 64 * 1024;    // LDS budget of the fused down + combine kernel
constexpr int kMB = 128;                      // bf16 MFMA path: rows (pairs) per M-block
constexpr int kNT = 256;                      // bf16 MFMA path: weight rows per work item

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
  // Host-resident layer (tiered placement): experts is the base of the HBM
  // expert cache and slot_of[e] (device, E + 1 entries, the shared expert
  // last) the slot holding expert e; null for a layer resident in HBM.
  const int32_t *slot_of;
};

// Address of expert e (E: the shared expert) of a layer.
__host__ __device__ inline const uint8_t *expert_base(const LayerDev &L, int e) {
  const int s = L.slot_of ? L.slot_of[e] : e;
  return L.experts + (size_t)s * L.expert_stride;
}

struct Dims {
  int d, f, E, k, T, n_shared;
};

struct UnionDev {
  int32_t *n_unique, *ids, *offsets, *pair_token, *pair_slot, *pair_of;
};

// Workspace carve-up (all offsets 256-byte aligned).
struct Workspace {
  size_t err;     // int32 error word set by kernels that reject a routing
  size_t n_unique, ids, offsets, pair_token, pair_slot, pair_of;  // union lists
  size_t logits;  // [Tmax][E] fp32
  size_t rpart;   // router partial sums for many tokens: [S][Tmax][E] fp32
  size_t h;       // [(Tmax*k + Tmax*n_shared)][f] fp32
  size_t y;       // [(Tmax*k + Tmax*n_shared)][d] fp32
  size_t xq, xs;  // fixed-point x: [Tmax][d/32][24] u32 digit words, [Tmax][d/16] fp32 scales
  size_t hq, hs;  // fixed-point h: [rows][f/32][24] u32, [rows][f/16] fp32
  size_t xb, hb;  // bf16 MFMA path: x rows in pair order [rows][d], h [rows][f], bf16
  size_t mblk, mcount;  // bf16 MFMA path: M-block lists (int4 entries, two classes of mblk_max) and their lengths
  size_t wslot;         // one-token path: gate weight of each slot in slot order
  int mblk_max;
  size_t bytes;
};

Workspace workspace_layout(int d, int f, int E, int k, int n_shared, int max_tokens);

// Kernel launchers (kernels.hip).  All enqueue on `s`, return hipError_t.
// Router with each expert row split over a block's 4 waves (T <= 16); xq/xs
// non-null: also encodes x for the fixed-point gate/up kernel.
hipError_t launch_router_split(const LayerDev &L, const Dims &D, const float *x, float *logits, uint32_t *xq,
                               float *xs, hipStream_t s);
// One token: the router applied to x = RMSNorm(r) (eps, unit weight) formed
// on the fly, with x written to xout and encoded into xq/xs; every value
// equals that of launch_rmsnorm followed by launch_router_split.
hipError_t launch_router_norm(const LayerDev &L, const Dims &D, const float *r, float eps, float *xout, float *logits,
                              uint32_t *xq, float *xs, hipStream_t s);
// Top-k of one token and, if U, its union lists (T == 1); top_p < 1 applies
// adaptive expert top-p (dropped slots: id -1, weight 0, pair_of -1).
// One token: the top-k and union lists of launch_topk_union1 and, in the same
// launch, the shared expert's fixed-point gate/up from the encoding xq/xs
// (into hq/hs row T*k, as launch_gateup_tok writes it).
bool shared_early_supported(const Dims &D);
hipError_t launch_topk_shared1(const float *logits, const Dims &D, int32_t *idx, float *w, const UnionDev *U,
                               float top_p, const LayerDev &L, const uint32_t *xq, const float *xs, uint32_t *hq,
                               float *hs, hipStream_t s);
// Router, top-k and (if U) union lists of one token in one launch, for E <= 32
// and d <= 2048 (the logits, selection and lists of the separate kernels).
bool route_one_small_supported(const Dims &D);
hipError_t launch_route_one_small(const LayerDev &L, const Dims &D, const float *x, float *logits, int32_t *idx,
                                  float *w, const UnionDev *U, float top_p, hipStream_t s);
// 2-4 tokens with union lists: launch_topk_union, and the shared expert's
// fixed-point gate/up for every token in the same launch (h rows T*k + t, as
// launch_gateup_tok writes them).
bool shared_early_multi_supported(const Dims &D);
hipError_t launch_topk_union_shared(const float *logits, const Dims &D, int32_t *idx, float *w, const UnionDev &U,
                                    int32_t *err, float top_p, const LayerDev &L, const uint32_t *xq,
                                    const float *xs, uint32_t *hq, float *hs, hipStream_t s);
hipError_t launch_topk_union1(const float *logits, const Dims &D, int32_t *idx, float *w, const UnionDev *U,
                              float top_p, hipStream_t s);
hipError_t launch_topk(const float *logits, const Dims &D, int32_t *idx, float *w, float top_p, hipStream_t s);
hipError_t launch_union(const int32_t *idx, const Dims &D, const UnionDev &U, int32_t *err, hipStream_t s);
// Top-k of 1..16 tokens and their union lists in one launch (the results of
// launch_topk followed by launch_union).
hipError_t launch_topk_union(const float *logits, const Dims &D, int32_t *idx, float *w, const UnionDev &U,
                             int32_t *err, float top_p, hipStream_t s);
hipError_t launch_gateup(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h,
                         hipStream_t s);
hipError_t launch_debug_gateup(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h,
                               float *g, float *u, hipStream_t s);
bool down_fusable(const Dims &D);
// One token on the narrow shapes (f < 2048) with k + shared <= 16: launch_down
// with fused set runs down and combine in one kernel.
bool narrow_dec_supported(const Dims &D);
// fused: y stays in LDS and the combine into `residual` happens in the same
// kernel; otherwise y is written to global memory for launch_combine.
hipError_t launch_down(const LayerDev &L, const Dims &D, const float *h, const UnionDev &U, float *y,
                       const float *w, float *residual, bool fused, hipStream_t s);
hipError_t launch_combine(const Dims &D, const float *w, const UnionDev &U, const float *y, float *residual,
                          hipStream_t s);
// Fixed-point activation path (d >= 2048 and f >= 2048).
bool fxp_supported(const Dims &D);
hipError_t launch_xquant(const float *x, int T, int K, uint32_t *xq, float *xs, hipStream_t s);
// Fixed-point gate/up for any T (one wave per tile and step, weights loaded
// once per call, tokens in chunks of 16); writes h's encoding to hq/hs and, for
// T == 1, each slot's gate weight (from w) to wslot[k + shared].
// skip_shared (one token, shared_early_supported): the shared expert's h is
// already there (launch_topk_shared1).
hipError_t launch_gateup_tok(const LayerDev &L, const Dims &D, const UnionDev &U, const int32_t *idx, const float *w,
                             const uint32_t *xq, const float *xs, uint32_t *hq, float *hs, float *wslot,
                             bool skip_shared, hipStream_t s);
// Fixed-point down for any T: y [T*k + T*shared][d] fp32 (combine in k_combine).
hipError_t launch_down_tok(const LayerDev &L, const Dims &D, const UnionDev &U, const uint32_t *hq, const float *hs,
                           float *y, hipStream_t s);
// Down + combine for one token when a down row is one step (f <= 2048) and
// k + shared <= 16 slots; slot gate weights from wslot.
bool down_dec_supported(const Dims &D);
// Down + combine for 2-4 tokens when a down row is one step (f <= 2048) and
// k + shared <= 16: a block per (token, output tile); the token's expert ids
// from idx, its gate weights from w; combine into the residual as
// launch_combine does.
bool down_dec_tok_supported(const Dims &D);
hipError_t launch_down_dec_tok(const LayerDev &L, const Dims &D, const uint32_t *hq, const float *hs,
                               const UnionDev &U, const int32_t *idx, const float *w, float *residual,
                               hipStream_t s);
hipError_t launch_down_dec(const LayerDev &L, const Dims &D, const uint32_t *hq, const float *hs, const UnionDev &U,
                           const float *wslot, float *residual, hipStream_t s);
// The fp32 dequantisation path for one token (d <= 8192, f a multiple of 16,
// down fusable, k + shared <= 16): gate/up writes h in a layout of its own
// that only launch_down_f32_dec reads, with h's sums over 16 columns in
// hsum ([rows][f/16]); down adds the combined output to residual.  Bits
// equal to launch_gateup + fused launch_down.
bool f32_dec_supported(const Dims &D);
hipError_t launch_gateup_f32_dec(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h,
                                 float *hsum, hipStream_t s);
hipError_t launch_down_f32_dec(const LayerDev &L, const Dims &D, const float *h, const float *hsum, const UnionDev &U,
                               const float *w, float *residual, hipStream_t s);
// The fp32 pair for 2-4 tokens (wide d and f, k + shared <= 16): gate/up per
// (pair, group), then down and combine per (token, tile) into the residual.
bool f32_dec_tok_supported(const Dims &D);
hipError_t launch_f32_dec_tok(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U,
                              const int32_t *idx, const float *w, float *h, float *hsum, float *residual,
                              hipStream_t s);
// Router for many tokens on the matrix cores (fp32), with S = router_splits(d)
// K-slices whose partials (part: [S][T][E]) are summed in slice order.
int router_splits(int d);
hipError_t launch_router_mfma(const LayerDev &L, const Dims &D, const float *x, float *part, float *logits,
                              hipStream_t s);
// bf16 MFMA path (prefill-shaped calls).
int mfma_max_entries(int T, int k, int E, int n_shared);
hipError_t launch_mblocks(const Dims &D, const UnionDev &U, int4 *list, int32_t *count, int max_entries,
                          hipStream_t s);
// xb [T][d] = bf16(x), one row per token.
hipError_t launch_gather_bf16(const float *x, const Dims &D, uint16_t *xb, hipStream_t s);
// A rows of the gate/up GEMM: pair p reads xb[pair_token[p]], shared row T*k + t
// reads xb[t].
hipError_t launch_gateup_mfma(const LayerDev &L, const Dims &D, const uint16_t *xb, const UnionDev &U,
                              const int4 *list, const int32_t *count, int max_entries, uint16_t *hb, hipStream_t s);
hipError_t launch_down_mfma(const LayerDev &L, const Dims &D, const uint16_t *hb, const int4 *list,
                            const int32_t *count, int max_entries, float *y, hipStream_t s);
hipError_t launch_rmsnorm(const float *r, int T, int d, float eps, float *x, hipStream_t s);
// Zeroes n 32-bit words with a kernel (not a memset node, so the call can sit
// in a captured graph).
hipError_t launch_zero_words(uint32_t *p, int n, hipStream_t s);

// Static device scratch of the allocation-free entry point (kernels.hip).
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
// Looks up the scratch array's address on `device`, which must be current;
// once per device, later calls return at once.
hipError_t static_scratch_init(int device);
// The address on `device`, or null before static_scratch_init succeeded there.
uint8_t *static_scratch(int device);
// int8 container, one token (fp32 dequantisation): h [rows][f] and y
// [rows][d] fp32 in the rows of the fixed-point path; the combine follows in
// launch_combine.
hipError_t launch_forward_i8(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h, float *y,
                             hipStream_t s);
// int8 container, one token (d <= 8192, f <= 2048, k + shared <= 16): the same
// results with the combine into `residual` in the down kernel (w: the gate
// weights).
bool i8_dec_supported(const Dims &D);
hipError_t launch_forward_i8_dec(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h,
                                 const float *w, float *residual, hipStream_t s);
// The int8 container for 2-16 tokens (as i8_dec_supported otherwise): gate/up
// per (4 h outputs, pair), then down and combine per (token, 8 rows).
bool i8_tok_supported(const Dims &D);
hipError_t launch_forward_i8_tok(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U,
                                 const int32_t *idx, float *h, const float *w, float *residual, hipStream_t s);
// Bytes of one expert in the int8 container (the canonical layout).
inline size_t expert_bytes_i8(int d, int f) {
  const size_t w = (size_t)d * (size_t)f;
  return 3 * (w + w / kGroup * 2);
}

}  // namespace colimoe
