// kernels.hip - HIP kernels for gfx950 (CDNA4) of the int4 routed-expert MoE
// layer.  Sources are cited by page title and section:
//   [A] "Colibrì: running a 744B MoE model on a laptop with 2400 lines of pure C"
//       (kechuai.cn article)
//   [P] "colibrì" project profile (gh.puless.com)
//   [D] "colibrì: 1300 lines of C, a 25 GB laptop, a 744-billion-parameter model"
//       (SSP GitHub Daily #091, jsqmd.com)
//
// Arithmetic: every float operation is written out (explicit fmaf, the file is
// built with -ffp-contract=off), so a token's result depends only on its own
// inputs and the code path, never on which other tokens share the call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "device_common.h"
#include "internal.h"

namespace colimoe {

// ------------------------------------------------------------------ helpers


// Scale of tile row `r` (0..7) from the 16-byte group record.
__device__ __forceinline__ float tile_scale(const uint4 &s, int r) {
  uint32_t w = (r >> 1) == 0 ? s.x : (r >> 1) == 1 ? s.y : (r >> 1) == 2 ? s.z : s.w;
  return (r & 1) ? half_hi(w) : half_lo(w);
}

// Dot product of 32 int4 weights (one 16-byte load of two's-complement
// nibbles) with 32 fp32 activations.  Each word is flipped to offset binary
// (n = q + 8, XOR 0x88888888), converted byte by byte, and the -8 * (sum of
// the activations), which the caller passes in as `nsx`, starts the sum:
//   sum_i (n_i - 8) x_i = sum_i q_i x_i.
// Byte b of word i holds columns 8i+2b (low nibble) and 8i+2b+1 (high).
// Even columns accumulate into alo, odd columns (read as 16 n) into ahi.
__device__ __forceinline__ float chunk_dot(const uint4 &w, const float4 *xv, float nsx) {
  const uint32_t ws[4] = {w.x ^ 0x88888888u, w.y ^ 0x88888888u, w.z ^ 0x88888888u, w.w ^ 0x88888888u};
  float alo = nsx, ahi = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = ws[i] & 0x0F0F0F0Fu, hi = ws[i] & 0xF0F0F0F0u;
    asm("" : "+v"(lo), "+v"(hi));  // keep the masks so byte conversions are single instructions
    const float4 xa = xv[2 * i], xb = xv[2 * i + 1];
    alo = __builtin_fmaf((float)(lo & 0xFFu), xa.x, alo);
    alo = __builtin_fmaf((float)((lo >> 8) & 0xFFu), xa.z, alo);
    alo = __builtin_fmaf((float)((lo >> 16) & 0xFFu), xb.x, alo);
    alo = __builtin_fmaf((float)(lo >> 24), xb.z, alo);
    ahi = __builtin_fmaf((float)(hi & 0xFFu), xa.y, ahi);
    ahi = __builtin_fmaf((float)((hi >> 8) & 0xFFu), xa.w, ahi);
    ahi = __builtin_fmaf((float)((hi >> 16) & 0xFFu), xb.y, ahi);
    ahi = __builtin_fmaf((float)(hi >> 24), xb.w, ahi);
  }
  return __builtin_fmaf(ahi, 0.0625f, alo);
}

// -8 * sum of the 32 activations of a chunk, summed in a fixed pairwise order.
__device__ __forceinline__ float neg8_sum(const float4 *xv) {
  float s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = (xv[i].x + xv[i].y) + (xv[i].z + xv[i].w);
  float t = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
  return -8.0f * t;
}

// DPP moves within 16-lane rows (lanes without a source read 0).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114;
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

// Value of lane l ^ 32 (one permlane32 swap).
__device__ __forceinline__ uint32_t xor32(uint32_t v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
// Value of lane l ^ 16 (one permlane16 swap).
__device__ __forceinline__ uint32_t xor16(uint32_t v) {
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (threadIdx.x & 16) ? r[0] : r[1];
}

// Sum over the 64 lanes of a wave, every lane receiving the same value.
// Fixed tree: l^32, l^16, then rotations by 8, 4, 2, 1 inside 16-lane rows.
__device__ __forceinline__ float wave_sum(float v) {
  v = v + bits_f(xor32(f_bits(v)));
  v = v + bits_f(xor16(f_bits(v)));
  v = v + bits_f(dpp<kRowRor8>(f_bits(v)));
  v = v + bits_f(dpp<kRowRor4>(f_bits(v)));
  v = v + bits_f(dpp<kRowRor2>(f_bits(v)));
  v = v + bits_f(dpp<kRowRor1>(f_bits(v)));
  return v;
}

// Maximum over the 64 lanes of a wave (unsigned 64-bit), every lane receiving it.
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint32_t lo, uint32_t hi) {
  const uint64_t b = ((uint64_t)hi << 32) | lo;
  return b > a ? b : a;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, xor32((uint32_t)v), xor32((uint32_t)(v >> 32)));
  v = max_u64(v, xor16((uint32_t)v), xor16((uint32_t)(v >> 32)));
  v = max_u64(v, dpp<kRowRor8>((uint32_t)v), dpp<kRowRor8>((uint32_t)(v >> 32)));
  v = max_u64(v, dpp<kRowRor4>((uint32_t)v), dpp<kRowRor4>((uint32_t)(v >> 32)));
  v = max_u64(v, dpp<kRowRor2>((uint32_t)v), dpp<kRowRor2>((uint32_t)(v >> 32)));
  v = max_u64(v, dpp<kRowRor1>((uint32_t)v), dpp<kRowRor1>((uint32_t)(v >> 32)));
  return v;
}

// Transposed reduction of 8 per-lane partials (one per tile row) across the
// 64 lanes of a wave.  Afterwards lane 8r+7 holds the full sum of row r.
// The tree is fixed: lanes l and l^32, then l^16, then l^8, then 4, 2, 1.
__device__ __forceinline__ float reduce8_rows(const float *p) {
  float q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    auto r = __builtin_amdgcn_permlane32_swap(f_bits(p[i]), f_bits(p[i + 4]), false, false);
    q[i] = bits_f(r[0]) + bits_f(r[1]);  // lanes 0-31: row i, lanes 32-63: row i+4
  }
  float t[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    auto r = __builtin_amdgcn_permlane16_swap(f_bits(q[i]), f_bits(q[i + 2]), false, false);
    t[i] = bits_f(r[0]) + bits_f(r[1]);  // 16-lane rows: i, i+2, i+4, i+6
  }
  const bool upper8 = (threadIdx.x & 8) != 0;
  const float keep = upper8 ? t[1] : t[0];
  const float send = upper8 ? t[0] : t[1];
  float v = keep + bits_f(dpp<kRowRor8>(f_bits(send)));
  v = v + bits_f(dpp<kRowShr4>(f_bits(v)));
  v = v + bits_f(dpp<kRowShr2>(f_bits(v)));
  v = v + bits_f(dpp<kRowShr1>(f_bits(v)));
  return v;
}

// Butterfly sum within aligned groups of `width` lanes (fixed tree).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v = v + __shfl_xor(v, o, 64);
  return v;
}

// ------------------------------------------------------------------- router
// A1 ([A] §1: a router picks 8 of the 256 experts): logits l[t][e] =
// sum_c R[e][c] x[t][c] + b[e] in fp32.  Up to 16 tokens: k_router_split
// below (one block per expert row); more tokens: the matrix-core kernel in
// kernels_mfma.hip.

// -------------------------------------------------------------------- top-k
// A2: the k largest logits, larger first, exact ties to the lower expert;
// gate weights = softmax over the selected logits.  One wave per token.

__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  uint32_t b = f_bits(v);
  if ((b & 0x7FFFFFFFu) == 0) b = 0;                                // +0 and -0 tie
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);  // monotone in v
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

// Selects for one token: k rounds of a wave-wide maximum over the keys; the
// selected logit is read back from its key (no memory access in the loop).
// Lane j keeps the j-th selected logit; gate weights are exp(v_j - v_0)
// divided by their sum, the sum taken by a fixed tree over lanes 0..15 and
// broadcast from lane 0.  Lane j writes entry j of idx and w (each if
// non-null) and the id to `lds_ids` (if given).  Every valid key is nonzero,
// so k <= E rounds always find one.
// Adaptive expert top-p ([D] key tuning parameters, "topp=0.7": an adaptive
// expert top-p that reads 30-40% fewer experts), for top_p < 1: lane j keeps
// its expert while the gate weights of the lanes before it sum to less than
// top_p (lane 0 always), the sum taken in lane order; kept lanes get the
// softmax over the kept logits (the same tree over lanes 0..15 with the
// dropped terms 0), dropped lanes write id -1 and weight 0.
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  return bits_f((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

template <int PER>
__device__ __forceinline__ void topk_token(const float *__restrict__ l, const Dims &D, int t,
                                           int32_t *__restrict__ idx, float *__restrict__ wout, int32_t *lds_ids,
                                           float top_p = 1.0f) {
  const int lane = threadIdx.x & 63;
  uint64_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < D.E ? topk_key(l[e], e) : 0ull;
  }
  float m = 0.0f, myv = 0.0f;
  int myid = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < D.k) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
      const float v = key_value(best);
      if (j == 0) m = v;
      if (lane == j) {
        myv = v;
        myid = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
      }
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (key[i] == best) key[i] = 0ull;
    }
  }
  const float ex = lane < D.k ? expf(myv - m) : 0.0f;
  float sum = ex + __shfl_xor(ex, 8, 64);
  sum = sum + __shfl_xor(sum, 4, 64);
  sum = sum + __shfl_xor(sum, 2, 64);
  sum = sum + __shfl_xor(sum, 1, 64);
  sum = bits_f(__builtin_amdgcn_readfirstlane(f_bits(sum)));
  float wj = ex / sum;
  if (top_p < 1.0f) {
    float before = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float wi = __shfl(wj, i, 64);
      if (i < lane) before = before + wi;
    }
    const bool keep = lane < D.k && (lane == 0 || before < top_p);
    const float exk = keep ? ex : 0.0f;
    float sk = exk + __shfl_xor(exk, 8, 64);
    sk = sk + __shfl_xor(sk, 4, 64);
    sk = sk + __shfl_xor(sk, 2, 64);
    sk = sk + __shfl_xor(sk, 1, 64);
    sk = bits_f(__builtin_amdgcn_readfirstlane(f_bits(sk)));
    wj = keep ? exk / sk : 0.0f;
    if (!keep) myid = -1;
  }
  if (lane < D.k) {
    if (idx) idx[(size_t)t * D.k + lane] = myid;
    if (wout) wout[(size_t)t * D.k + lane] = wj;
    if (lds_ids) lds_ids[t * D.k + lane] = myid;
  }
}

template <int PER>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ logits, Dims D, int32_t *__restrict__ idx,
                                              float *__restrict__ wout, float top_p) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t < D.T) topk_token<PER>(logits + (size_t)t * D.E, D, t, idx, wout, nullptr, top_p);
}

// -------------------------------------------------------------------- union
// A3 ([A] §2, batch-union: batched positions read each unique expert once):
// distinct experts ascending, and every (token, slot) pair grouped by expert
// in token order.  One wave; ranks come from per-expert lane masks in LDS, so
// the result is independent of timing.  Invalid routings (expert out of
// range, or an expert twice in one token) produce an empty union and set *err.
// idx may point to LDS (the top-k's copy of the routing, up to 16 tokens).
// LDS: masks[E] u64 (8-byte aligned), counts[E], running[E], one flag.

// An expert id of -1 in a routing marks a slot dropped by expert top-p: it
// gets no pair (pair_of -1) and is not read; any other id outside [0, E) is
// an invalid routing.
constexpr int kDropped = -1;

__host__ __device__ inline size_t union_lds_bytes(int E) { return (size_t)E * 8 + (size_t)(2 * E + 1) * 4; }

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ void union_wave(const int32_t *__restrict__ idx, const Dims &D, const UnionDev &U,
                           int32_t *__restrict__ err, unsigned long long *masks) {
  const int E = D.E, k = D.k, T = D.T;
  int32_t *counts = (int32_t *)(masks + E);
  int32_t *running = counts + E;
  int32_t &bad = running[E];
  const int lane = threadIdx.x & 63;
  if (lane == 0) bad = 0;
  for (int e = lane; e < E; e += 64) {
    counts[e] = 0;
    masks[e] = 0ull;
  }
  wave_lds_sync();
  for (int t = lane; t < T; t += 64) {
    // the token's k ids first (one round of loads), then the checks
    int ee[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) ee[j] = j < k ? idx[(size_t)t * k + j] : kDropped;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = ee[j];
      if (j >= k || e == kDropped) continue;
      bool ok = e >= 0 && e < E;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < j) ok = ok && ee[i] != e;
      if (!ok)
        bad = 1;
      else
        atomicAdd(&counts[e], 1);
    }
  }
  wave_lds_sync();
  if (bad) {
    if (lane == 0) {
      *U.n_unique = 0;
      U.offsets[0] = 0;
      atomicOr(err, 1);
    }
    return;
  }
  // exclusive scans of counts and of (counts > 0), lane-blocked
  const int per = (E + 63) / 64;
  const int e0 = lane * per, e1 = min(E, e0 + per);
  int csum = 0, nsum = 0;
  for (int e = e0; e < e1; ++e) {
    csum += counts[e];
    nsum += counts[e] > 0;
  }
  int cinc = csum, ninc = nsum;
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(cinc, o, 64), b = __shfl_up(ninc, o, 64);
    if (lane >= o) {
      cinc += a;
      ninc += b;
    }
  }
  int cb = cinc - csum, nb = ninc - nsum;
  for (int e = e0; e < e1; ++e) {
    running[e] = cb;
    if (counts[e] > 0) {
      U.ids[nb] = e;
      U.offsets[nb] = cb;
      ++nb;
    }
    cb += counts[e];
  }
  if (lane == 63) {
    *U.n_unique = ninc;
    U.offsets[ninc] = cinc;
  }
  wave_lds_sync();
  for (int t0 = 0; t0 < T; t0 += 64) {
    const int t = t0 + lane;
    const bool act = t < T;
    int ee[16];
    unsigned long long mm[16];
    int rr[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      ee[j] = act && j < k ? idx[(size_t)t * k + j] : kDropped;
      if (ee[j] != kDropped) atomicOr(&masks[ee[j]], 1ull << lane);
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      rr[j] = -1;
      if (ee[j] != kDropped) {
        mm[j] = masks[ee[j]];
        rr[j] = __popcll(mm[j] & ((1ull << lane) - 1ull));
        const int p = running[ee[j]] + rr[j];
        U.pair_token[p] = t;
        U.pair_slot[p] = j;
        U.pair_of[(size_t)t * k + j] = p;
      } else if (act && j < k) {
        U.pair_of[(size_t)t * k + j] = -1;
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (rr[j] == 0) {
        running[ee[j]] += __popcll(mm[j]);
        masks[ee[j]] = 0ull;
      }
    wave_lds_sync();
  }
}

__global__ __launch_bounds__(64) void k_union(const int32_t *__restrict__ idx, Dims D, UnionDev U,
                                              int32_t *__restrict__ err) {
  extern __shared__ __align__(16) unsigned long long union_lds[];
  union_wave(idx, D, U, err, union_lds);
}

// Union for many tokens: the W waves of one block each take a contiguous
// segment of tokens.  Per-(segment, expert) counts, prefixed over segments in
// wave order and offset by each expert's start, give every wave the position
// of its first pair of each expert, so the scatter (one wave per segment,
// 64-token chunks ranked with lane masks as above) keeps token order inside
// every expert.  Same lists as the one-wave kernel.
// LDS: masks[W][E] u64, segc[W][E], counts[E], start[E], one flag.
__host__ __device__ inline size_t union_multi_lds_bytes(int E, int W) {
  return (size_t)W * E * 8 + ((size_t)W * E + 2 * (size_t)E + 1) * 4;
}

__global__ __launch_bounds__(1024) void k_union_multi(const int32_t *__restrict__ idx, Dims D, UnionDev U,
                                                      int32_t *__restrict__ err) {
  extern __shared__ __align__(16) unsigned long long union_lds[];
  const int E = D.E, k = D.k, T = D.T;
  const int W = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  unsigned long long *masks = union_lds;
  int32_t *segc = (int32_t *)(masks + (size_t)W * E);
  int32_t *counts = segc + (size_t)W * E;
  int32_t *start = counts + E;
  int32_t &bad = start[E];
  for (int i = threadIdx.x; i < W * E; i += blockDim.x) {
    masks[i] = 0ull;
    segc[i] = 0;
  }
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const int seg = (T + W - 1) / W;
  const int t_lo = min(T, wave * seg), t_hi = min(T, t_lo + seg);
  int32_t *mycount = segc + (size_t)wave * E;
  for (int t = t_lo + lane; t < t_hi; t += 64) {
    // the token's k ids in registers first (one round of loads), then the
    // checks: distinct and in range
    int ee[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) ee[j] = j < k ? idx[(size_t)t * k + j] : kDropped;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = ee[j];
      if (j >= k || e == kDropped) continue;
      bool ok = e >= 0 && e < E;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < j) ok = ok && ee[i] != e;
      if (!ok)
        bad = 1;
      else
        atomicAdd(&mycount[e], 1);
    }
  }
  __syncthreads();
  if (bad) {
    if (threadIdx.x == 0) {
      *U.n_unique = 0;
      U.offsets[0] = 0;
      atomicOr(err, 1);
    }
    return;
  }
  // per expert: exclusive prefix over segments (wave order) and the total
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int w = 0; w < W; ++w) {
      const int c = segc[(size_t)w * E + e];
      segc[(size_t)w * E + e] = run;
      run += c;
    }
    counts[e] = run;
  }
  __syncthreads();
  if (wave == 0) {  // exclusive scans of counts and of (counts > 0), lane-blocked
    const int per = (E + 63) / 64;
    const int e0 = lane * per, e1 = min(E, e0 + per);
    int csum = 0, nsum = 0;
    for (int e = e0; e < e1; ++e) {
      csum += counts[e];
      nsum += counts[e] > 0;
    }
    int cinc = csum, ninc = nsum;
    for (int o = 1; o < 64; o <<= 1) {
      const int a = __shfl_up(cinc, o, 64), b = __shfl_up(ninc, o, 64);
      if (lane >= o) {
        cinc += a;
        ninc += b;
      }
    }
    int cb = cinc - csum, nb = ninc - nsum;
    for (int e = e0; e < e1; ++e) {
      start[e] = cb;
      if (counts[e] > 0) {
        U.ids[nb] = e;
        U.offsets[nb] = cb;
        ++nb;
      }
      cb += counts[e];
    }
    if (lane == 63) {
      *U.n_unique = ninc;
      U.offsets[ninc] = cinc;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < W * E; i += blockDim.x) segc[i] += start[i % E];
  __syncthreads();
  // scatter: wave w over its segment, running positions in segc[w][*]
  unsigned long long *mymask = masks + (size_t)wave * E;
  for (int c0 = t_lo; c0 < t_hi; c0 += 64) {
    const int t = c0 + lane;
    const bool act = t < t_hi;
    int ee[16];
    unsigned long long mm[16];
    int rr[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      ee[j] = act && j < k ? idx[(size_t)t * k + j] : kDropped;
      if (ee[j] != kDropped) atomicOr(&mymask[ee[j]], 1ull << lane);
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      rr[j] = -1;
      if (ee[j] != kDropped) {
        mm[j] = mymask[ee[j]];
        rr[j] = __popcll(mm[j] & ((1ull << lane) - 1ull));
        const int p = mycount[ee[j]] + rr[j];
        U.pair_token[p] = t;
        U.pair_slot[p] = j;
        U.pair_of[(size_t)t * k + j] = p;
      } else if (act && j < k) {
        U.pair_of[(size_t)t * k + j] = -1;
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (rr[j] == 0) {
        mycount[ee[j]] += __popcll(mm[j]);
        mymask[ee[j]] = 0ull;
      }
    wave_lds_sync();
  }
}

// ----------------------------------------------------------- expert GEMVs
// A4-A6: W[r][c] = q[r][c] * s[r][c/64] ([P] "conservative correctness":
// int4, group size 64), dequantised to fp32 and multiplied in fp32 ([D] §4,
// highlight 4: at batch 1, f32 rather than integer arithmetic), fp32
// accumulation.  Work is cut into 8-row tiles; each lane handles 32-column
// chunks (one 16-byte load per row), each wave one 64-chunk step of a tile
// (8 rows x 1 KB, contiguous in the device layout).  A step's weights, once
// in registers, are applied to up to MT of the expert's tokens, so each
// weight is read from HBM once per call when no expert has more than MT
// tokens.  Per token and row the operations (chunk dots, scale fmas, lane
// and wave reduction trees) do not depend on MT or on the other tokens:
// batched and one-at-a-time results are bit-identical.

__device__ __forceinline__ void load_step(const uint8_t *__restrict__ nib, const uint8_t *__restrict__ sc, int tile,
                                          int K, int c, uint4 (&W)[kTileRows], uint4 &S) {
  const int G = K / kGroup;
  S = *(const uint4 *)(sc + ((size_t)tile * G + (c >> 1)) * 16);
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) W[r] = *(const uint4 *)(nib + chunk_offset(tile, K, c, r));
}

// acc[r] = fma(s_r, chunk dot, acc[r]) for the 8 rows of a step, the
// chunk's 32 activations in xv.
__device__ __forceinline__ void step_accumulate_xv(const uint4 (&W)[kTileRows], const uint4 &S, const float4 (&xv)[8],
                                                   float (&acc)[kTileRows]) {
  const float nsx = neg8_sum(xv);
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) acc[r] = __builtin_fmaf(tile_scale(S, r), chunk_dot(W[r], xv, nsx), acc[r]);
}

// The same for one token's activation row xrow, chunk c.
__device__ __forceinline__ void step_accumulate(const uint4 (&W)[kTileRows], const uint4 &S,
                                                const float *__restrict__ xrow, int c, float (&acc)[kTileRows]) {
  float4 xv[8];
  const float4 *src = (const float4 *)(xrow + (size_t)kChunk * c);
#pragma unroll
  for (int v = 0; v < 8; ++v) xv[v] = src[v];
  step_accumulate_xv(W, S, xv, acc);
}

// Gate/up for K = d >= 2048: a block of NW = ceil(d/2048) waves per work item
// (unique expert slot, tile of 4 gate + 4 up rows); wave w handles chunks
// 64w..64w+63 of the 8 rows, the block sums the waves' row totals in wave
// order and writes h = SiLU(g) * u per pair.  Slot nu (after the routed
// experts) is the shared expert with all T tokens ([D] §3).
template <int MT>
__global__ __launch_bounds__(512) void k_gateup_wide(LayerDev L, Dims D, const float *__restrict__ x, UnionDev U,
                                                      float *__restrict__ h, float *__restrict__ gdbg,
                                                      float *__restrict__ udbg) {
  __shared__ float red[8][MT][kTileRows];
  const int nw = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int C = D.d / kChunk, tiles = D.f / 4;
  const int nu = clamp_nu(U.n_unique, D);
  const int items = (nu + D.n_shared) * tiles;
  const ExpertLayout EL = expert_layout(D.d, D.f);
  const int c = lane + 64 * wave;
  const bool active = c < C;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int s = item / tiles, ti = item - s * tiles;
    int e, p0, p1;
    if (!resolve_slot(D, U, nu, s, e, p0, p1)) continue;
    const uint8_t *base = expert_base(L, e);
    uint4 W[kTileRows], S;
    if (active) load_step(base + EL.gu_nib, base + EL.gu_sc, ti, D.d, c, W, S);
    for (int pg = p0; pg < p1; pg += MT) {
      const int mcount = min(MT, p1 - pg);
      float acc[MT][kTileRows];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int r = 0; r < kTileRows; ++r) acc[m][r] = 0.0f;
        if (m < mcount && active) {
          int t, orow;
          slot_token(D, U, nu, s, pg + m, t, orow);
          step_accumulate(W, S, x + (size_t)t * D.d, c, acc[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < mcount) {
          const float v = reduce8_rows(acc[m]);
          if ((lane & 7) == 7) red[wave][m][lane >> 3] = v;
        }
      __syncthreads();
      if ((int)threadIdx.x < mcount * 4) {
        const int m = threadIdx.x >> 2, r = threadIdx.x & 3;
        float g = red[0][m][r], u = red[0][m][r + 4];
        for (int w2 = 1; w2 < nw; ++w2) {
          g = g + red[w2][m][r];
          u = u + red[w2][m][r + 4];
        }
        int t, orow;
        slot_token(D, U, nu, s, pg + m, t, orow);
        if (orow >= 0) {
          const size_t o = (size_t)orow * D.f + (size_t)ti * 4 + r;
          h[o] = silu_f(g) * u;
          if (gdbg) {
            gdbg[o] = g;
            udbg[o] = u;
          }
        }
      }
      __syncthreads();
    }
  }
}

// The fp32 dequantisation path's one-token pair of kernels ([D] §4
// highlight 4: f32 at batch 1).  Their h rows use a chunk-interleaved
// layout: element 32c + 4v + i of a row (chunk c, float4 v of the chunk) is
// stored at (v C + c) 4 + i, C = f / 32, so that the down kernel's lane c
// reads float4 v of its chunk in one coalesced load per v (a plain row
// would give every lane its own 128-byte line).  The layout is private to
// the pair: no other kernel reads or writes it.
__device__ __forceinline__ size_t h_ilv(int col, int C) {
  return (size_t)((((col & 31) >> 2) * C + (col >> 5)) * 4 + (col & 3));
}

// Gate/up: a block of 4 waves per (slot, 4 TPW tiles); wave w takes tiles
// TPW w .. TPW w + TPW - 1, each tile's NS steps (d <= 8192) one after the
// other, the next step's weights loading while the current step computes.
// x is staged once per block in LDS, 36 floats per 32-float chunk so that a
// wave's 16-byte reads of one float4 of 64 chunks fall in distinct banks,
// with each chunk's neg8_sum in the pad.  Per h row the operations are
// those of k_gateup_wide (the lane's chunk, fma(scale, chunk_dot, 0), the
// fixed 8-row tree, the steps added in order, SiLU(g) * u): the bits are
// those of the batched fp32 kernels.
constexpr int kXPad = 36;      // LDS floats per 32-activation chunk
constexpr int kF32DecTPW = 1;  // tiles per wave
// PAIRS (2-4 tokens): a block per (pair, group) instead of (slot, group), on
// the pair's token, items ordered and spread over the XCDs as in
// k_gateup_pairs; h rows are the pairs' (routed pair p, shared T*k + t).
template <int NS, int TPW, bool PAIRS>
__global__ __launch_bounds__(256) void k_gateup_f32_dec(LayerDev L, Dims D, const float *__restrict__ x, UnionDev U,
                                                        float *__restrict__ h, float *__restrict__ hsum,
                                                        const int32_t *__restrict__ idx, int n_items) {
  __shared__ __attribute__((aligned(16))) float xl[NS * 64 * kXPad];
  __shared__ float s4[4];    // each wave's float4 sum of h
  __shared__ int slot_s[3];  // expert, output row, token
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int C = D.d / kChunk, groups = D.f / (16 * TPW);
  int grp;
  if (PAIRS) {
    const int per = (int)gridDim.x / 8;
    const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (item >= n_items) return;  // block-uniform
    const int tk = D.T * D.k, P = tk + D.T * D.n_shared;
    grp = item / P;
    const int p = item - grp * P;
    if (threadIdx.x == 0) {
      int e = -1, t = 0;
      if (p < tk) {
        const int nu = clamp_nu(U.n_unique, D);
        int np = U.offsets[nu];
        np = np < 0 ? 0 : (np > tk ? tk : np);
        t = U.pair_token[p];
        const int j = U.pair_slot[p];
        if (p < np && t >= 0 && t < D.T && j >= 0 && j < D.k) {
          e = idx[(size_t)t * D.k + j];
          if (e < 0 || e >= D.E) e = -1;
        }
      } else {
        t = p - tk;
        e = D.E;
      }
      slot_s[0] = e;
      slot_s[1] = p;
      slot_s[2] = t;
    }
  } else {
    const int s = blockIdx.x / groups;
    grp = blockIdx.x - s * groups;
    if (threadIdx.x == 0) {
      const int nu = clamp_nu(U.n_unique, D);
      int e = -1, p0 = 0, p1 = 0;
      if (s < nu || (s == nu && D.n_shared)) {
        if (!resolve_slot(D, U, nu, s, e, p0, p1) || p1 <= p0) e = -1;
      }
      slot_s[0] = e;
      slot_s[1] = s < nu ? p0 : D.T * D.k;
      slot_s[2] = 0;
    }
  }
  __syncthreads();
  const int e = slot_s[0], orow = slot_s[1];
  if (e < 0) return;  // block-uniform
  x += (size_t)slot_s[2] * D.d;
  const ExpertLayout EL = expert_layout(D.d, D.f);
  const uint8_t *base = expert_base(L, e);
  // weights through buffer loads (the lane's offset in a VGPR, the rest in
  // the scalar offset); a lane past the row end reads the row's last chunk
  // and its sums are replaced by 0
  const __amdgpu_buffer_rsrc_t rn = wave_rsrc(base + EL.gu_nib, (uint32_t)(EL.gu_sc - EL.gu_nib));
  const __amdgpu_buffer_rsrc_t rs = wave_rsrc(base + EL.gu_sc, (uint32_t)(EL.dn_nib - EL.gu_sc));
  const int tile0 = grp * 4 * TPW + wave * TPW;
  constexpr int kItems = NS * TPW;
  uint4 Wb[2][kTileRows], Sb[2];
  auto issue = [&](int it, uint4(&W)[kTileRows], uint4 &S) {
    const int ti = tile0 + it / NS, st = it % NS;
    const int width = C - 64 * st < 64 ? C - 64 * st : 64;
    const int cl = lane < width ? lane : width - 1;
    const int tb = ti * kTileRows * (D.d / 2) + st * (kTileRows * 64 * 16);
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rn, cl * 16, tb + r * width * 16, 0);
      W[r] = make_uint4(t.x, t.y, t.z, t.w);
    }
    const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rs, (cl >> 1) * 16, (ti * (D.d / kGroup) + 32 * st) * 16, 0);
    S = make_uint4(t.x, t.y, t.z, t.w);
  };
  issue(0, Wb[0], Sb[0]);
  // x into LDS; each float4's sum, then the chunk's 8 sums in neg8_sum's
  // tree (the 8 float4s of a chunk sit in 8 consecutive lanes; a + b is
  // b + a exactly, so the shifted partners give the same sums)
  for (int q = threadIdx.x; q < C * 8; q += blockDim.x) {
    const float4 xq = ((const float4 *)x)[q];
    *(float4 *)&xl[(q >> 3) * kXPad + (q & 7) * 4] = xq;
    float v = (xq.x + xq.y) + (xq.z + xq.w);
    v = v + bits_f(dpp<kRowShr1>(f_bits(v)));
    v = v + bits_f(dpp<kRowShr2>(f_bits(v)));
    v = v + bits_f(dpp<kRowShr4>(f_bits(v)));
    if ((q & 7) == 7) xl[(q >> 3) * kXPad + 32] = -8.0f * v;
  }
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    if (it + 1 < kItems) issue(it + 1, Wb[(it + 1) & 1], Sb[(it + 1) & 1]);
    const uint4(&W)[kTileRows] = Wb[it & 1];
    const uint4 &S = Sb[it & 1];
    const int ti = tile0 + it / NS, st = it % NS;
    const int width = C - 64 * st < 64 ? C - 64 * st : 64;
    const bool live = lane < width;
    const float *xc = &xl[(64 * st + (live ? lane : width - 1)) * kXPad];
    // chunk_dot of the 8 rows, a word's 8 columns at a time: per row the
    // same two chains (even columns from -8 sum x, odd from 0), same order
    float alo[kTileRows], ahi[kTileRows];
    const float nsx = xc[32];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      alo[r] = nsx;
      ahi[r] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 xa = *(const float4 *)&xc[8 * i], xb = *(const float4 *)&xc[8 * i + 4];
#pragma unroll
      for (int r = 0; r < kTileRows; ++r) {
        const uint32_t wi = (i == 0 ? W[r].x : i == 1 ? W[r].y : i == 2 ? W[r].z : W[r].w) ^ 0x88888888u;
        uint32_t lo = wi & 0x0F0F0F0Fu, hi = wi & 0xF0F0F0F0u;
        asm("" : "+v"(lo), "+v"(hi));
        alo[r] = __builtin_fmaf((float)(lo & 0xFFu), xa.x, alo[r]);
        alo[r] = __builtin_fmaf((float)((lo >> 8) & 0xFFu), xa.z, alo[r]);
        alo[r] = __builtin_fmaf((float)((lo >> 16) & 0xFFu), xb.x, alo[r]);
        alo[r] = __builtin_fmaf((float)(lo >> 24), xb.z, alo[r]);
        ahi[r] = __builtin_fmaf((float)(hi & 0xFFu), xa.y, ahi[r]);
        ahi[r] = __builtin_fmaf((float)((hi >> 8) & 0xFFu), xa.w, ahi[r]);
        ahi[r] = __builtin_fmaf((float)((hi >> 16) & 0xFFu), xb.y, ahi[r]);
        ahi[r] = __builtin_fmaf((float)(hi >> 24), xb.w, ahi[r]);
      }
      // the word's sums are due here: one word's masks and activations
      // live at a time
#pragma unroll
      for (int r = 0; r < kTileRows; ++r) asm volatile("" : "+v"(alo[r]), "+v"(ahi[r]));
    }
    float acc[kTileRows];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r)
      acc[r] = live ? __builtin_fmaf(tile_scale(S, r), __builtin_fmaf(ahi[r], 0.0625f, alo[r]), 0.0f) : 0.0f;
    const float v = reduce8_rows(acc);  // row r of this step at lane 8r + 7
    tot = st == 0 ? v : tot + v;
    if (st == NS - 1) {
      // gate row r (lane 8r + 7) meets up row r + 4 (lane 8r + 39)
      const float u = bits_f(xor32(f_bits(tot)));
      const float hv = silu_f(tot) * u;
      if ((lane & 7) == 7 && lane < 32) h[(size_t)orow * D.f + h_ilv(ti * 4 + (lane >> 3), D.f / kChunk)] = hv;
      // the sum of this float4 of h, in neg8_sum's order
      const float a = __shfl(hv, 7, 64), b = __shfl(hv, 15, 64), c = __shfl(hv, 23, 64), d = __shfl(hv, 31, 64);
      if (lane == 0) s4[wave] = (a + b) + (c + d);
    }
  }
  // the block's 4 float4s are half a 32-column chunk: its first-level sum
  __syncthreads();
  if (threadIdx.x == 0) hsum[(size_t)orow * (D.f / 16) + grp] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
}

// A7 for one 8-row output tile, y of every pair in LDS: per token and row,
// the routed experts in ascending expert id (ascending pair index, since the
// union lists are grouped by expert) weighted by w, then the shared expert.
__device__ __forceinline__ void combine_tile(const Dims &D, const UnionDev &U, int nu, const float *__restrict__ w,
                                             const float *ylds, float *__restrict__ residual, int ti) {
  const int tk = D.T * D.k;
  for (int q = threadIdx.x; q < D.T * kTileRows; q += blockDim.x) {
    const int t = q >> 3, r = q & 7;
    float *rp = residual + (size_t)t * D.d + (size_t)ti * kTileRows + r;
    float acc = *rp;
    if (nu > 0) {
      int pj[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) pj[j] = j < D.k ? U.pair_of[(size_t)t * D.k + j] : 0x7FFFFFFF;
      int prev = -1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i < D.k) {
          int best = 0x7FFFFFFF, bj = 0;
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (pj[j] > prev && pj[j] < best) {
              best = pj[j];
              bj = j;
            }
          if (best < tk) acc = __builtin_fmaf(w[(size_t)t * D.k + bj], ylds[(size_t)best * kTileRows + r], acc);
          prev = best;
        }
      }
    }
    if (D.n_shared) acc = acc + ylds[((size_t)tk + t) * kTileRows + r];
    *rp = acc;
  }
}

// Down projection for K = f >= 2048 with the combine fused in: a block owns an
// 8-row output tile; its waves take the call's slots round-robin, run all
// chunk steps of their slot (y = Wd h for each of the slot's tokens) and
// leave y in LDS; then the block adds, per token and row, the routed experts
// in ascending expert id (ascending pair index) weighted by w, then the
// shared expert, into the residual.  FUSED == false writes y to global
// memory instead (k_combine finishes), for calls too large for LDS.
template <int MT, bool FUSED, int NWMAX>
__global__ __launch_bounds__(64 * NWMAX) void k_down_wide(LayerDev L, Dims D, const float *__restrict__ h, UnionDev U,
                                                    float *__restrict__ y, const float *__restrict__ w,
                                                    float *__restrict__ residual) {
  extern __shared__ float ylds[];  // [T*k + T*n_shared][8] when FUSED
  const int nw = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int C = D.f / kChunk, tiles = D.d / kTileRows;
  const int nu = clamp_nu(U.n_unique, D);
  const int slots = nu + D.n_shared;
  const int tk = D.T * D.k;
  const ExpertLayout EL = expert_layout(D.d, D.f);
  for (int ti = blockIdx.x; ti < tiles; ti += gridDim.x) {
    for (int s = wave; s < slots; s += nw) {
      int e, p0, p1;
      if (!resolve_slot(D, U, nu, s, e, p0, p1)) continue;
      const uint8_t *base = expert_base(L, e);
      for (int pg = p0; pg < p1; pg += MT) {
        const int mcount = min(MT, p1 - pg);
        float acc[MT][kTileRows];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int r = 0; r < kTileRows; ++r) acc[m][r] = 0.0f;
        for (int c = lane; c < ((C + 63) & ~63); c += 64) {
          if (c < C) {
            uint4 W[kTileRows], S;
            load_step(base + EL.dn_nib, base + EL.dn_sc, ti, D.f, c, W, S);
#pragma unroll
            for (int m = 0; m < MT; ++m)
              if (m < mcount) {
                const int orow = (s < nu) ? pg + m : tk + pg + m;
                step_accumulate(W, S, h + (size_t)orow * D.f, c, acc[m]);
              }
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < mcount) {
            const float v = reduce8_rows(acc[m]);
            if ((lane & 7) == 7) {
              const int orow = (s < nu) ? pg + m : tk + pg + m;
              if (FUSED)
                ylds[(size_t)orow * kTileRows + (lane >> 3)] = v;
              else
                y[(size_t)orow * D.d + (size_t)ti * kTileRows + (lane >> 3)] = v;
            }
          }
      }
    }
    if (FUSED) {
      __syncthreads();
      combine_tile(D, U, nu, w, ylds, residual, ti);
      __syncthreads();
    }
  }
}

// ------------------------------------------------ fixed-point activations
// A4-A6 on the decode path with exact int4 arithmetic.  Each group of 16
// consecutive activations (x for gate/up, h for down) is encoded as signed
// integers X_i = rint(v_i 2^(22-E)) with 2^E > max|v| over the group, so
// |X_i| <= 2^22 and |v_i - X_i 2^(E-22)| <= 2^(E-23) <= 2^-22 max|v|.  X is
// split into six signed base-16 digits (each in [-8, 7]) packed eight to a
// word in the weights' nibble order, so one v_dot8_i32_i4 multiplies 8 int4
// weights by 8 digits exactly.  Per 16 columns and row: six digit-plane
// dot products (exact int32), recombined as sum_k 16^k a_k (exact in
// int32, rounded once to fp32), scaled by s_row * 2^(E-22) and
// accumulated in fp32 along the row.  The weights are the canonical
// two's-complement nibbles, read as they are.

// Group exponent: the smallest E with max|v| < 2^E (at least -100), and the
// group's scale 2^(E-22).  mb is the bit pattern of max|v|, taken as an
// integer maximum over the |v| patterns, so a NaN or an infinity in the
// group wins it.  Such a group gets a NaN scale (every output it enters is
// NaN, as on the fp32 path: no silent change of the result) and its values
// are encoded as zeros (fin = false), so no non-finite value reaches the
// integer conversion.
__device__ __forceinline__ int fxp_exponent(uint32_t mb, float &scale, bool &fin) {
  fin = mb < 0x7F800000u;
  const float mx = bits_f(fin ? mb : 0u);
  int E = mx > 0.0f ? ilogbf(mx) + 1 : 0;
  E = E < -100 ? -100 : E;
  scale = fin ? ldexpf(1.0f, E - 22) : __builtin_nanf("");
  return E;
}

// Encodes 16 values; words[2k + w] holds digit plane k of columns 8w..8w+7.
__device__ __forceinline__ void quant16(const float *v, uint32_t *words, float &scale) {
  uint32_t mb = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) mb = max(mb, f_bits(fabsf(v[i])));
  bool fin;
  const int E = fxp_exponent(mb, scale, fin);
  const float up = ldexpf(1.0f, 22 - E);
#pragma unroll
  for (int k = 0; k < 12; ++k) words[k] = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t B = (uint32_t)((int)__builtin_rintf((fin ? v[i] : 0.0f) * up) + 0x888888);
#pragma unroll
    for (int k = 0; k < 6; ++k) words[2 * k + (i >> 3)] |= (((B >> (4 * k)) & 15u) ^ 8u) << (4 * (i & 7));
  }
}

// acc += s * sum over a 32-column chunk of q_i * v_i, with the chunk's digit
// words dg[24] ([half][plane][2]) and half-group scales xs[2].
__device__ __forceinline__ float fxp_chunk(const uint4 &w, const uint32_t *dg, const float *xs, float s, float acc) {
  const uint32_t wh[2][2] = {{w.x, w.y}, {w.z, w.w}};
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    // V = sum_k 16^k a_k by Horner from the top plane down, each plane's two
    // dot8s accumulating into 16 * (the planes above): exact in int32, since
    // |V| = |sum_i q_i X_i| <= 16 * 8 * 2^22 = 2^29; rounded once to fp32
    int t = 0;
#pragma unroll
    for (int k = 5; k >= 0; --k) {
      t = __builtin_amdgcn_sdot8((int)wh[hf][0], (int)dg[hf * 12 + 2 * k], t * 16, false);
      t = __builtin_amdgcn_sdot8((int)wh[hf][1], (int)dg[hf * 12 + 2 * k + 1], t, false);
    }
    const float V = (float)t;
    acc = __builtin_fmaf(s * xs[hf], V, acc);
  }
  return acc;
}

// Digit words and scales of chunk c of activation row `row` (K columns).
__device__ __forceinline__ void load_digits(const uint32_t *__restrict__ q, const float *__restrict__ qs, int row, int K,
                                            int c, uint32_t (&dg)[kDigitWords], float (&xs)[2]) {
  const uint4 *src = (const uint4 *)(q + ((size_t)row * (K / kChunk) + c) * kDigitWords);
#pragma unroll
  for (int i = 0; i < kDigitWords / 4; ++i) {
    const uint4 v = src[i];
    dg[4 * i] = v.x;
    dg[4 * i + 1] = v.y;
    dg[4 * i + 2] = v.z;
    dg[4 * i + 3] = v.w;
  }
  const float2 sv = *(const float2 *)(qs + (size_t)row * (K / 16) + 2 * c);
  xs[0] = sv.x;
  xs[1] = sv.y;
}

__device__ __forceinline__ void fxp_apply(const uint4 (&W)[kTileRows], const uint4 &S, const uint32_t (&dg)[kDigitWords],
                                          const float (&xs)[2], float (&acc)[kTileRows]) {
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) acc[r] = fxp_chunk(W[r], dg, xs, tile_scale(S, r), acc[r]);
}

__device__ __forceinline__ void fxp_step(const uint4 (&W)[kTileRows], const uint4 &S, const uint32_t *__restrict__ q,
                                         const float *__restrict__ qs, int row, int K, int c,
                                         float (&acc)[kTileRows]) {
  uint32_t dg[kDigitWords];
  float xs[2];
  load_digits(q, qs, row, K, c, dg, xs);
  fxp_apply(W, S, dg, xs, acc);
}

// Encodes T rows of x (K columns each) for the gate/up kernel; one lane per
// 16-column group.
__device__ __forceinline__ void xquant_group(const float *__restrict__ x, int K, int g, uint32_t *__restrict__ q,
                                             float *__restrict__ qs) {
  const int gpr = K / 16;
  const int t = g / gpr, gi = g - t * gpr;
  float v[16];
  const float4 *src = (const float4 *)(x + (size_t)t * K + (size_t)gi * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 f = src[i];
    v[4 * i] = f.x;
    v[4 * i + 1] = f.y;
    v[4 * i + 2] = f.z;
    v[4 * i + 3] = f.w;
  }
  uint32_t words[12];
  float scale;
  quant16(v, words, scale);
  uint4 *dst = (uint4 *)(q + ((size_t)t * (K / kChunk) + (gi >> 1)) * kDigitWords + (gi & 1) * 12);
  dst[0] = make_uint4(words[0], words[1], words[2], words[3]);
  dst[1] = make_uint4(words[4], words[5], words[6], words[7]);
  dst[2] = make_uint4(words[8], words[9], words[10], words[11]);
  qs[(size_t)t * gpr + gi] = scale;
}

// As xquant_group for one row whose values are x * inv.
__device__ __forceinline__ void xquant_group_scaled(const float *__restrict__ x, int K, int g, float inv, uint32_t *__restrict__ q,
                                             float *__restrict__ qs) {
  const int gpr = K / 16;
  const int t = g / gpr, gi = g - t * gpr;
  float v[16];
  const float4 *src = (const float4 *)(x + (size_t)t * K + (size_t)gi * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 f = src[i];
    v[4 * i] = f.x * inv;
    v[4 * i + 1] = f.y * inv;
    v[4 * i + 2] = f.z * inv;
    v[4 * i + 3] = f.w * inv;
  }
  uint32_t words[12];
  float scale;
  quant16(v, words, scale);
  uint4 *dst = (uint4 *)(q + ((size_t)t * (K / kChunk) + (gi >> 1)) * kDigitWords + (gi & 1) * 12);
  dst[0] = make_uint4(words[0], words[1], words[2], words[3]);
  dst[1] = make_uint4(words[4], words[5], words[6], words[7]);
  dst[2] = make_uint4(words[8], words[9], words[10], words[11]);
  qs[(size_t)t * gpr + gi] = scale;
}

__global__ __launch_bounds__(256) void k_xquant(const float *__restrict__ x, int T, int K, uint32_t *__restrict__ q,
                                                float *__restrict__ qs) {
  const int groups = T * (K / 16);
  for (int g = blockIdx.x * 256 + threadIdx.x; g < groups; g += gridDim.x * 256) xquant_group(x, K, g, q, qs);
}

// Fixed-point GEMVs for any number of tokens.  A block owns 4 tiles (32
// weight rows) of one slot and has, per tile, up to 4 waves that split the
// row's steps (64 chunks each; wave sg takes steps sg, sg + 4, ...).  Each
// wave loads its weights once and applies them to every token of the slot
// (16 at a time, token rows staged in LDS).  Per token and step a lane's
// contribution is formed from zero, reduced across the wave by the fixed
// tree of reduce8_rows, and the per-step row values are added in step order:
// v = ((R_0 + R_1) + R_2) + ...  This order is the same whatever T is, so a
// token gives bit-identical results alone or batched.
constexpr int kTokChunk = 16;

template <int SPW, bool ONE>
__device__ __forceinline__ void tile_tokens(const uint8_t *__restrict__ nib, const uint8_t *__restrict__ scp, int ti,
                                            int K, int sg, int wpt, const int *tok, int mc,
                                            const uint32_t *__restrict__ q, const float *__restrict__ qs,
                                            float *red /* [NS][kTokChunk][8] of this tile */) {
  const int lane = threadIdx.x & 63;
  const int C = K / kChunk, NS = (C + 63) / 64;
  uint4 W[SPW][kTileRows], S[SPW];
#pragma unroll
  for (int k = 0; k < SPW; ++k) {
    const int j = sg + wpt * k, c = lane + 64 * j;
    if (j < NS && c < C) load_step(nib, scp, ti, K, c, W[k], S[k]);
  }
  for (int m = 0; m < (ONE ? 1 : mc); ++m) {
    const int row = tok[m];
#pragma unroll
    for (int k = 0; k < SPW; ++k) {
      const int j = sg + wpt * k, c = lane + 64 * j;
      if (j < NS) {
        float acc[kTileRows];
#pragma unroll
        for (int r = 0; r < kTileRows; ++r) acc[r] = 0.0f;
        if (c < C) fxp_step(W[k], S[k], q, qs, row, K, c, acc);
        const float v = reduce8_rows(acc);
        if ((lane & 7) == 7) red[((size_t)j * kTokChunk + m) * kTileRows + (lane >> 3)] = v;
      }
    }
  }
}

// Gate/up: block = (slot, 16 h rows = 4 tiles); after each chunk of tokens the
// block forms h = SiLU(g) * u per token and encodes its 16 values for the down
// kernel.  For T == 1 the first block of each slot also records the slot's
// gate weight in wslot (slot order, 1 for the shared expert).
// WPT waves per tile (block = 4 * WPT waves).
template <int SPW, bool ONE, int WPT>
__global__ __launch_bounds__(256 * WPT) void k_gateup_tok(LayerDev L, Dims D, UnionDev U, const float *__restrict__ w,
                                                     const uint32_t *__restrict__ xq, const float *__restrict__ xs,
                                                     uint32_t *__restrict__ hq, float *__restrict__ hs,
                                                     float *__restrict__ wslot) {
  extern __shared__ float red[];  // [4 tiles][NS][kTokChunk][8]
  __shared__ int slot_s[4];       // expert, p0, p1, nu
  __shared__ int tok_s[kTokChunk], orow_s[kTokChunk];
  __shared__ float hv[kTokChunk][16];
  __shared__ uint32_t hw[kTokChunk][12];
  __shared__ float hsc[kTokChunk];
  const int wave = threadIdx.x >> 6;
  const int C = D.d / kChunk, NS = (C + 63) / 64, wpt = WPT;
  const int quads = D.f / 16;
  const int s = blockIdx.x / quads, qd = blockIdx.x - s * quads;
  const int tt = wave / wpt, sg = wave - tt * wpt, ti = qd * 4 + tt;
  if (threadIdx.x == 0) {
    const int nu = clamp_nu(U.n_unique, D);
    int e = -1, p0 = 0, p1 = 0;
    if (s < nu || (s == nu && D.n_shared)) {
      if (!resolve_slot(D, U, nu, s, e, p0, p1) || p1 <= p0) e = -1;
    }
    slot_s[0] = e;
    slot_s[1] = p0;
    slot_s[2] = p1;
    slot_s[3] = nu;
    if (D.T == 1 && qd == 0 && e >= 0) {
      float f = 1.0f;
      if (s < nu) {
        int js = U.pair_slot[p0];
        js = js < 0 ? 0 : (js >= D.k ? D.k - 1 : js);  // caller-supplied lists stay in bounds
        f = w[js];
      }
      wslot[s] = f;
    }
  }
  __syncthreads();
  const int e = slot_s[0], p0 = slot_s[1], p1 = slot_s[2], nu = slot_s[3];
  if (e < 0) return;  // block-uniform
  const ExpertLayout EL = expert_layout(D.d, D.f);
  const uint8_t *base = expert_base(L, e);
  for (int pg = p0; pg < p1; pg += kTokChunk) {
    const int mc = min(kTokChunk, p1 - pg);
    if ((int)threadIdx.x < mc) {
      int t, orow;
      slot_token(D, U, nu, s, pg + threadIdx.x, t, orow);
      tok_s[threadIdx.x] = t;
      orow_s[threadIdx.x] = orow;
    }
    if ((int)threadIdx.x < kTokChunk * 12) hw[threadIdx.x / 12][threadIdx.x % 12] = 0u;
    __syncthreads();
    tile_tokens<SPW, ONE>(base + EL.gu_nib, base + EL.gu_sc, ti, D.d, sg, wpt, tok_s, mc, xq, xs,
                     red + (size_t)tt * NS * kTokChunk * kTileRows);
    __syncthreads();
    // h for (token m, h row i): tile i/4, gate row i%4, up row i%4 + 4
    if ((int)threadIdx.x < mc * 16) {
      const int m = threadIdx.x >> 4, i = threadIdx.x & 15;
      const float *rt = red + (size_t)(i >> 2) * NS * kTokChunk * kTileRows + (size_t)m * kTileRows;
      float g = rt[i & 3], u = rt[(i & 3) + 4];
      for (int j = 1; j < NS; ++j) {
        g = g + rt[(size_t)j * kTokChunk * kTileRows + (i & 3)];
        u = u + rt[(size_t)j * kTokChunk * kTileRows + (i & 3) + 4];
      }
      hv[m][i] = silu_f(g) * u;
    }
    __syncthreads();
    // encode each token's 16 h values (one 16-lane row per token)
    if ((int)threadIdx.x < kTokChunk * 16) {
      const int m = threadIdx.x >> 4, i = threadIdx.x & 15;
      const float v = m < mc ? hv[m][i] : 0.0f;
      uint32_t mb = f_bits(fabsf(v));
      mb = max(mb, dpp<kRowRor8>(mb));
      mb = max(mb, dpp<kRowRor4>(mb));
      mb = max(mb, dpp<kRowRor2>(mb));
      mb = max(mb, dpp<kRowRor1>(mb));
      float sc;
      bool fin;
      const int E = fxp_exponent(mb, sc, fin);
      if (m < mc) {
        const uint32_t B = (uint32_t)((int)__builtin_rintf((fin ? v : 0.0f) * ldexpf(1.0f, 22 - E)) + 0x888888);
#pragma unroll
        for (int k = 0; k < 6; ++k) atomicOr(&hw[m][2 * k + (i >> 3)], (((B >> (4 * k)) & 15u) ^ 8u) << (4 * (i & 7)));
        if (i == 0) hsc[m] = sc;
      }
    }
    __syncthreads();
    if ((int)threadIdx.x < mc * 12) {
      const int m = threadIdx.x / 12, wd = threadIdx.x % 12;
      const int orow = orow_s[m];
      if (orow >= 0) {
        hq[((size_t)orow * (D.f / kChunk) + (qd >> 1)) * kDigitWords + (qd & 1) * 12 + wd] = hw[m][wd];
        if (wd == 0) hs[(size_t)orow * (D.f / 16) + qd] = hsc[m];
      }
    }
    __syncthreads();
  }
}

// Gate/up for one token, up to 4 steps per row (d <= 8192): one wave per
// (tile, step), the same operations as k_gateup_tok with a single token, in
// a lean form that keeps two blocks resident per CU.  One block: 16 h rows
// (4 tiles, quad qd) of expert e into output row orow.
template <int NS>
__device__ __forceinline__ void gateup_one_quad(const LayerDev &L, const Dims &D, int e, int orow, int qd, int xrow,
                                                const uint32_t *__restrict__ xq, const float *__restrict__ xs,
                                                uint32_t *__restrict__ hq, float *__restrict__ hs) {
  __shared__ float red[4][NS][kTileRows];
  __shared__ uint32_t hw[12];
  __shared__ float hsc;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int C = D.d / kChunk;
  const int tt = wave / NS, st = wave - tt * NS;
  const int ti = qd * 4 + tt, c = lane + 64 * st;
  if (threadIdx.x < 12) hw[threadIdx.x] = 0u;
  const ExpertLayout EL = expert_layout(D.d, D.f);
  const uint8_t *base = expert_base(L, e);
  float acc[kTileRows];
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) acc[r] = 0.0f;
  if (c < C) {
    uint4 W[kTileRows], S;
    load_step(base + EL.gu_nib, base + EL.gu_sc, ti, D.d, c, W, S);
    uint32_t dg[kDigitWords];
    float dsc[2];
    load_digits(xq, xs, xrow, D.d, c, dg, dsc);
    // loads issued: from here the wave outranks waves of newer blocks still
    // issuing theirs, so blocks whose data has arrived finish and retire
    // sooner (measured: gate/up 0.2-0.4 us faster; the same in the down
    // kernel was slower)
    __builtin_amdgcn_s_setprio(2);
    fxp_apply(W, S, dg, dsc, acc);
  }
  const float v = reduce8_rows(acc);
  if ((lane & 7) == 7) red[tt][st][lane >> 3] = v;
  __syncthreads();
  if (threadIdx.x < 16) {
    const int i = threadIdx.x, t4 = i >> 2, r = i & 3;
    float g = red[t4][0][r], u = red[t4][0][r + 4];
#pragma unroll
    for (int j = 1; j < NS; ++j) {
      g = g + red[t4][j][r];
      u = u + red[t4][j][r + 4];
    }
    const float hval = silu_f(g) * u;
    uint32_t mb = f_bits(fabsf(hval));
    mb = max(mb, dpp<kRowRor8>(mb));
    mb = max(mb, dpp<kRowRor4>(mb));
    mb = max(mb, dpp<kRowRor2>(mb));
    mb = max(mb, dpp<kRowRor1>(mb));
    float sc;
    bool fin;
    const int E = fxp_exponent(mb, sc, fin);
    const uint32_t B = (uint32_t)((int)__builtin_rintf((fin ? hval : 0.0f) * ldexpf(1.0f, 22 - E)) + 0x888888);
#pragma unroll
    for (int k = 0; k < 6; ++k) atomicOr(&hw[2 * k + (i >> 3)], (((B >> (4 * k)) & 15u) ^ 8u) << (4 * (i & 7)));
    if (i == 0) hsc = sc;
  }
  __syncthreads();
  if (threadIdx.x < 12) {
    hq[((size_t)orow * (D.f / kChunk) + (qd >> 1)) * kDigitWords + (qd & 1) * 12 + threadIdx.x] = hw[threadIdx.x];
    if (threadIdx.x == 0) hs[(size_t)orow * (D.f / 16) + qd] = hsc;
  }
}

// Routed slots (and, unless skip_shared, the shared expert after them): a
// block per (slot, quad); the first quad of a routed slot records the slot's
// gate weight in wslot.
template <int NS>
__global__ __launch_bounds__(256 * NS) void k_gateup_one(LayerDev L, Dims D, UnionDev U, const float *__restrict__ w,
                                                         const uint32_t *__restrict__ xq,
                                                         const float *__restrict__ xs, uint32_t *__restrict__ hq,
                                                         float *__restrict__ hs, float *__restrict__ wslot,
                                                         int skip_shared) {
  __shared__ int slot_s[2];  // expert, output row
  const int quads = D.f / 16;
  const int s = blockIdx.x / quads, qd = blockIdx.x - s * quads;
  if (threadIdx.x == 0) {
    const int nu = clamp_nu(U.n_unique, D);
    int e = -1, p0 = 0, p1 = 0;
    if (s < nu || (s == nu && D.n_shared && !skip_shared)) {
      if (!resolve_slot(D, U, nu, s, e, p0, p1) || p1 <= p0) e = -1;
    }
    slot_s[0] = e;
    slot_s[1] = s < nu ? p0 : D.k;
    if (qd == 0 && e >= 0) {
      float f = 1.0f;
      if (s < nu) {
        int js = U.pair_slot[p0];
        js = js < 0 ? 0 : (js >= D.k ? D.k - 1 : js);  // caller-supplied lists stay in bounds
        f = w[js];
      }
      wslot[s] = f;
    }
  }
  __syncthreads();
  const int e = slot_s[0], orow = slot_s[1];
  if (e < 0) return;  // block-uniform
  gateup_one_quad<NS>(L, D, e, orow, qd, 0, xq, xs, hq, hs);
}

// 2-16 tokens: a block per (pair, quad), the one-token block code on the
// pair's token, so each token's h has the bits of the token alone.  Items are
// (quad, pair) with the pair fastest; the block ids are remapped so that each
// XCD takes one contiguous range of items, which puts the pairs of one expert
// (consecutive in the union lists) and quad on one L2 at about the same time:
// the weights come from HBM once and the other pairs' reads hit that L2.  A
// routed pair's expert is idx[token][top-k position]; pairs past the list's
// count (dropped by expert top-p) exit.  The items hold the shared expert's T
// rows after the routed pairs, unless the top-k launch has written them.
template <int NS>
__global__ __launch_bounds__(256 * NS) void k_gateup_pairs(LayerDev L, Dims D, UnionDev U,
                                                           const int32_t *__restrict__ idx,
                                                           const uint32_t *__restrict__ xq,
                                                           const float *__restrict__ xs, uint32_t *__restrict__ hq,
                                                           float *__restrict__ hs, int n_items) {
  __shared__ int pr_s[3];  // expert, token, output row
  const int per = (int)gridDim.x / 8;
  const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (item >= n_items) return;  // block-uniform
  const int tk = D.T * D.k, P = n_items / (D.f / 16);  // pairs per quad: tk, plus T shared rows unless done
  const int qd = item / P, p = item - qd * P;
  if (threadIdx.x == 0) {
    int e = -1, t = 0;
    if (p < tk) {
      const int nu = clamp_nu(U.n_unique, D);
      int np = U.offsets[nu];
      np = np < 0 ? 0 : (np > tk ? tk : np);
      t = U.pair_token[p];
      const int j = U.pair_slot[p];
      if (p < np && t >= 0 && t < D.T && j >= 0 && j < D.k) {
        e = idx[(size_t)t * D.k + j];
        if (e < 0 || e >= D.E) e = -1;
      }
    } else {
      t = p - tk;
      e = D.E;
    }
    pr_s[0] = e;
    pr_s[1] = t;
    pr_s[2] = p;
  }
  __syncthreads();
  const int e = pr_s[0];
  if (e < 0) return;  // block-uniform
  gateup_one_quad<NS>(L, D, e, pr_s[2], qd, pr_s[1], xq, xs, hq, hs);
}

constexpr int kPairsMaxT = 16;   // tokens up to which gate/up runs per pair
constexpr int kDownTokMaxT = 4;  // tokens up to which down runs per token (with the combine)
constexpr int kF32TokMaxT = 16;  // the same for the fp32 pair
// tokens up to which the shared gate/up rides in the top-k launch (at 16 the
// shared expert's 16 token rows outlast the selection: +25 us of top-k launch
// for -15 us of gate/up)
constexpr int kSharedEarlyMaxT = 4;

// Down: block = (slot, 4 output tiles = 32 rows); y[output row of the pair]
// for each of the slot's pairs (the shared expert: rows T*k + t).  The
// combine runs afterwards in k_combine (or, for one token, in k_down_dec1).
template <int SPW, bool ONE, int WPT>
__global__ __launch_bounds__(256 * WPT) void k_down_tok(LayerDev L, Dims D, UnionDev U, const uint32_t *__restrict__ hq,
                                                   const float *__restrict__ hs, float *__restrict__ y) {
  extern __shared__ float red[];  // [4 tiles][NS][kTokChunk][8]
  __shared__ int slot_s[4];
  __shared__ int row_s[kTokChunk];
  const int wave = threadIdx.x >> 6;
  const int C = D.f / kChunk, NS = (C + 63) / 64, wpt = WPT;
  const int groups = D.d / 32;
  const int s = blockIdx.x / groups, qd = blockIdx.x - s * groups;
  const int tt = wave / wpt, sg = wave - tt * wpt, ti = qd * 4 + tt;
  if (threadIdx.x == 0) {
    const int nu = clamp_nu(U.n_unique, D);
    int e = -1, p0 = 0, p1 = 0;
    if (s < nu || (s == nu && D.n_shared)) {
      if (!resolve_slot(D, U, nu, s, e, p0, p1) || p1 <= p0) e = -1;
    }
    slot_s[0] = e;
    slot_s[1] = p0;
    slot_s[2] = p1;
    slot_s[3] = nu;
  }
  __syncthreads();
  const int e = slot_s[0], p0 = slot_s[1], p1 = slot_s[2], nu = slot_s[3];
  if (e < 0) return;  // block-uniform
  const ExpertLayout EL = expert_layout(D.d, D.f);
  const uint8_t *base = expert_base(L, e);
  const int tk = D.T * D.k;
  for (int pg = p0; pg < p1; pg += kTokChunk) {
    const int mc = min(kTokChunk, p1 - pg);
    if ((int)threadIdx.x < mc) row_s[threadIdx.x] = s < nu ? pg + threadIdx.x : tk + pg + threadIdx.x;
    __syncthreads();
    tile_tokens<SPW, ONE>(base + EL.dn_nib, base + EL.dn_sc, ti, D.f, sg, wpt, row_s, mc, hq, hs,
                     red + (size_t)tt * NS * kTokChunk * kTileRows);
    __syncthreads();
    for (int q = threadIdx.x; q < mc * 32; q += blockDim.x) {
      const int m = q >> 5, i = q & 31;  // output row 32*qd + i
      const float *rt = red + (size_t)(i >> 3) * NS * kTokChunk * kTileRows + (size_t)m * kTileRows + (i & 7);
      float v = rt[0];
      for (int j = 1; j < NS; ++j) v = v + rt[(size_t)j * kTokChunk * kTileRows];
      y[(size_t)row_s[m] * D.d + (size_t)qd * 32 + i] = v;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------ decode (T == 1) path
// One token: every slot holds exactly one pair (pair index = slot for the
// routed experts, T*k for the shared one).  The kernels below keep each wave
// streaming with the next step's loads in flight while it computes the
// current one; per row they perform exactly the operations of the general
// fixed-point kernels above (same chunk order, same reduction trees, same
// combine order), so their results are bit-identical to them.

// Dot products of one wave's quarter row r with tokens t0..t0+G-1 (rows past T
// are clamped to T-1, computed and dropped); part[t][wave] = the wave's sum.
template <int G>
__device__ __forceinline__ void router_tokens(const float4 (&r)[16], const float *__restrict__ x, const Dims &D,
                                              int wave, int lane, int q4, float (*part)[4]) {
  for (int t0 = 0; t0 < D.T; t0 += G) {
    float acc[G];
#pragma unroll
    for (int u = 0; u < G; ++u) acc[u] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = 4 * lane + 256 * i;
      if (c < q4) {
#pragma unroll
        for (int u = 0; u < G; ++u) {
          const int t = t0 + u < D.T ? t0 + u : D.T - 1;
          const float4 xv = *(const float4 *)(x + (size_t)t * D.d + (size_t)wave * q4 + c);
          acc[u] = __builtin_fmaf(r[i].x, xv.x, acc[u]);
          acc[u] = __builtin_fmaf(r[i].y, xv.y, acc[u]);
          acc[u] = __builtin_fmaf(r[i].z, xv.z, acc[u]);
          acc[u] = __builtin_fmaf(r[i].w, xv.w, acc[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const float v = wave_sum(acc[u]);
      if (lane == 0 && t0 + u < D.T) part[t0 + u][wave] = v;
    }
  }
}

// One token whose x is r * inv (formed per element as it is read), with the
// operations and order of router_tokens<1>.
__device__ __forceinline__ void router_tokens_scaled(const float4 (&rw)[16], const float *__restrict__ rres,
                                                     const Dims &D, int wave, int lane, int q4, float inv,
                                                     float (*part)[4]) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = 4 * lane + 256 * i;
    if (c < q4) {
      const float4 rv = *(const float4 *)(rres + (size_t)wave * q4 + c);
      const float4 xv = make_float4(rv.x * inv, rv.y * inv, rv.z * inv, rv.w * inv);
      acc = __builtin_fmaf(rw[i].x, xv.x, acc);
      acc = __builtin_fmaf(rw[i].y, xv.y, acc);
      acc = __builtin_fmaf(rw[i].z, xv.z, acc);
      acc = __builtin_fmaf(rw[i].w, xv.w, acc);
    }
  }
  const float v = wave_sum(acc);
  if (lane == 0) part[0][wave] = v;
}

// x = r * inv of one token with inv = 1 / sqrt(mean(r^2) + eps): the sum of
// squares in exactly the order of k_rmsnorm's 512 threads (thread t sums the
// float4 columns t, t + 512, ... in order; each wave's tree; the 8 wave sums
// by a fixed tree), emulated by a block of 256 threads (thread t plays t and
// t + 256, whose waves are w and w + 4), so inv is the same bits.
__device__ __forceinline__ float rms_inv_256(const float *__restrict__ r, int d, float eps, float *part8) {
  const float4 *rr = (const float4 *)r;
  const int n4 = d / 4, t = threadIdx.x;
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c0 = t + 512 * i, c1 = t + 256 + 512 * i;
    const float4 v0 = c0 < n4 ? rr[c0] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 v1 = c1 < n4 ? rr[c1] : make_float4(0.f, 0.f, 0.f, 0.f);
    a0 = __builtin_fmaf(v0.x, v0.x, a0);
    a0 = __builtin_fmaf(v0.y, v0.y, a0);
    a0 = __builtin_fmaf(v0.z, v0.z, a0);
    a0 = __builtin_fmaf(v0.w, v0.w, a0);
    a1 = __builtin_fmaf(v1.x, v1.x, a1);
    a1 = __builtin_fmaf(v1.y, v1.y, a1);
    a1 = __builtin_fmaf(v1.z, v1.z, a1);
    a1 = __builtin_fmaf(v1.w, v1.w, a1);
  }
  a0 = wave_sum(a0);
  a1 = wave_sum(a1);
  if ((t & 63) == 0) {
    part8[t >> 6] = a0;
    part8[(t >> 6) + 4] = a1;
  }
  __syncthreads();
  const float ss = ((part8[0] + part8[1]) + (part8[2] + part8[3])) + ((part8[4] + part8[5]) + (part8[6] + part8[7]));
  return 1.0f / sqrtf(ss / (float)d + eps);
}

// Router with the d columns split over the 4 waves of a block, one block per
// expert row, up to 16 tokens.  Each wave keeps its quarter of the row in
// registers and applies it to every token; the 4 partial sums of a token are
// added in wave order.  A token's logit does not depend on T.  NORM (one
// token): x is RMSNorm(r) formed on the fly (every block computes the same
// inv; x = r * inv wherever x is read), and x_out receives it.
template <bool NORM>
__global__ __launch_bounds__(256) void k_router_split(LayerDev L, Dims D, const float *__restrict__ x,
                                                      float *__restrict__ logits, uint32_t *__restrict__ xq,
                                                      float *__restrict__ xs, float eps, float *__restrict__ xout) {
  __shared__ float part[kRouteSplitMaxT][4];
  __shared__ float part8[8];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x;
  const int q4 = D.d / 4;  // columns per wave (d is a multiple of 64, at most 16384)
  const float *row = L.router + (size_t)e * D.d + (size_t)wave * q4;
  float4 r[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = 4 * lane + 256 * i;
    r[i] = c < q4 ? *(const float4 *)(row + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (NORM) {
    const float inv = rms_inv_256(x, D.d, eps, part8);
    for (int c = blockIdx.x * 256 + threadIdx.x; c < D.d / 4; c += gridDim.x * 256) {
      const float4 v = ((const float4 *)x)[c];
      ((float4 *)xout)[c] = make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
    }
    const int groups = D.d / 16;
    for (int g = blockIdx.x * 256 + threadIdx.x; g < groups; g += gridDim.x * 256) xquant_group_scaled(x, D.d, g, inv, xq, xs);
    router_tokens_scaled(r, x, D, wave, lane, q4, inv, part);
  } else {
    if (xq) {  // fixed-point encoding of x for the gate/up kernel, while the row is in flight
      const int groups = D.T * (D.d / 16);
      for (int g = blockIdx.x * 256 + threadIdx.x; g < groups; g += gridDim.x * 256) xquant_group(x, D.d, g, xq, xs);
    }
    // one token alone, two or three together, or tokens four or eight at a
    // time so their loads and reductions overlap; per token the operations
    // and their order are the same
    if (D.T == 1)
      router_tokens<1>(r, x, D, wave, lane, q4, part);
    else if (D.T == 2)
      router_tokens<2>(r, x, D, wave, lane, q4, part);
    else if (D.T == 3)
      router_tokens<3>(r, x, D, wave, lane, q4, part);
    else if (D.T < 8)
      router_tokens<4>(r, x, D, wave, lane, q4, part);
    else
      router_tokens<8>(r, x, D, wave, lane, q4, part);
  }
  __syncthreads();
  if (threadIdx.x < D.T)
    logits[(size_t)threadIdx.x * D.E + e] =
        ((part[threadIdx.x][0] + part[threadIdx.x][1]) + part[threadIdx.x][2]) + part[threadIdx.x][3] + L.bias[e];
}

// Union lists of one token from its k expert ids (in LDS; distinct, or -1 for
// a slot dropped by expert top-p): the kept ids ascending, one pair each,
// pair_slot = the id's position in the top-k, pair_of = -1 for a dropped slot.
__device__ __forceinline__ void union_one_token(const int32_t *ids, const Dims &D, const UnionDev &U) {
  const int j = threadIdx.x & 63;
  if (j < D.k) {
    int m = 0;
    for (int i = 0; i < D.k; ++i) m += ids[i] >= 0;
    const int e = ids[j];
    if (e >= 0) {
      int rank = 0;
      for (int i = 0; i < D.k; ++i) rank += ids[i] >= 0 && ids[i] < e;
      U.ids[rank] = e;
      U.offsets[rank] = rank;
      U.pair_token[rank] = 0;
      U.pair_slot[rank] = j;
      U.pair_of[j] = rank;
    } else {
      U.pair_of[j] = -1;
    }
    if (j == 0) {
      *U.n_unique = m;
      U.offsets[m] = m;
    }
  }
}

// Top-k of one token plus its union lists.
template <int PER>
__global__ __launch_bounds__(64) void k_topk_union1(const float *__restrict__ logits, Dims D,
                                                    int32_t *__restrict__ idx, float *__restrict__ wout, UnionDev U,
                                                    int with_union, float top_p) {
  __shared__ int32_t ids[16];
  topk_token<PER>(logits, D, 0, idx, wout, ids, top_p);
  wave_lds_sync();
  if (with_union) union_one_token(ids, D, U);
}

// Router, top-k and union lists of one token in one block, for small routers
// (E <= 32, d <= 2048; at 64 experts the one block's row loads cost more than
// the launch it saves).  Wave group g (4 waves) takes rows g, g + 4, ...,
// wave w of the group the quarter of the columns k_router_split gives it;
// every row's loads are issued before any arithmetic, then per row the fmas
// in router_tokens<1>'s order, the wave sum and the 4 partial sums added in
// wave order: the logits are k_router_split's bits.  Wave 0 then selects as
// k_topk_union1 does.
constexpr int kRouteOneMaxE = 32;
template <int NF, int PER>
__global__ __launch_bounds__(1024) void k_route_one_small(LayerDev L, Dims D, const float *__restrict__ x,
                                                          float *__restrict__ logits, int32_t *__restrict__ idx,
                                                          float *__restrict__ wout, UnionDev U, int with_union,
                                                          float top_p) {
  constexpr int RB = kRouteOneMaxE / 4;  // rows per wave group at most
  __shared__ float part[kRouteOneMaxE][4];
  __shared__ float lg[kRouteOneMaxE];
  __shared__ int32_t ids[16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g4 = wave >> 2, w4 = wave & 3, q4 = D.d / 4;
  float4 xv[NF], rr[RB][NF];
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    const int c = 4 * lane + 256 * i;
    xv[i] = c < q4 ? *(const float4 *)(x + (size_t)w4 * q4 + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int e = g4 + 4 * b;
    const float *row = L.router + (size_t)(e < D.E ? e : 0) * D.d + (size_t)w4 * q4;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int c = 4 * lane + 256 * i;
      rr[b][i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < D.E && c < q4) rr[b][i] = *(const float4 *)(row + c);  // rows past E load nothing
    }
  }
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int e = g4 + 4 * b;
    if (e < D.E) {  // wave-uniform
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int c = 4 * lane + 256 * i;
        if (c < q4) {
          acc = __builtin_fmaf(rr[b][i].x, xv[i].x, acc);
          acc = __builtin_fmaf(rr[b][i].y, xv[i].y, acc);
          acc = __builtin_fmaf(rr[b][i].z, xv[i].z, acc);
          acc = __builtin_fmaf(rr[b][i].w, xv[i].w, acc);
        }
      }
      const float v = wave_sum(acc);
      if (lane == 0) part[e][w4] = v;
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < D.E) {
    const int e = threadIdx.x;
    const float v = ((part[e][0] + part[e][1]) + part[e][2]) + part[e][3] + L.bias[e];
    lg[e] = v;
    logits[e] = v;
  }
  __syncthreads();
  if (wave == 0) {
    topk_token<PER>(lg, D, 0, idx, wout, ids, top_p);
    wave_lds_sync();
    if (with_union) union_one_token(ids, D, U);
  }
}

// Top-k of one token plus its union lists (block 0, as k_topk_union1), and
// beside it the shared expert's gate/up (blocks 1..f/16, one quad each, as
// k_gateup_one): the shared expert does not depend on the routing, so its
// weights stream while the selection runs.
template <int PER, int NS>
__global__ __launch_bounds__(256 * NS) void k_topk_shared1(const float *__restrict__ logits, Dims D,
                                                           int32_t *__restrict__ idx, float *__restrict__ wout,
                                                           UnionDev U, int with_union, float top_p, LayerDev L,
                                                           const uint32_t *__restrict__ xq,
                                                           const float *__restrict__ xs, uint32_t *__restrict__ hq,
                                                           float *__restrict__ hs) {
  __shared__ int32_t ids[16];
  if (blockIdx.x == 0) {
    if (threadIdx.x < 64) {
      topk_token<PER>(logits, D, 0, idx, wout, ids, top_p);
      wave_lds_sync();
      if (with_union) union_one_token(ids, D, U);
    }
    return;
  }
  gateup_one_quad<NS>(L, D, D.E, D.T * D.k, (int)blockIdx.x - 1, 0, xq, xs, hq, hs);
}

// Down + combine for one token when a down row is one step (f <= 2048): a
// block of one wave per slot owns one 8-row output tile; every wave issues its
// slot's weights and digits at once and leaves the slot's 8 outputs in LDS;
// wave 0 folds them into the residual in slot order (routed experts by
// ascending id weighted by their gate weight, taken from wslot as recorded by
// the gate/up kernel, then the shared expert), as the general kernels do.
// The weights come through buffer loads (one lane offset, the row in the
// scalar offset), which keeps the kernel small enough in registers for three
// blocks per CU: the whole grid of d/8 blocks is resident at once.  Every
// lane computes (a lane past the row end reads a valid chunk and its result
// is replaced by 0), so no load sits behind a branch.
constexpr int kDecMaxSlots = 16;  // slots of the one-token down kernel (one wave each)

// One wave of the one-step down kernels: the 8 rows of output tile ti of
// expert e (when ok) against h row hrow, reduced by the fixed tree into
// out[0..8).  Every lane computes (a lane past the row end reads a valid
// chunk and its result is replaced by 0), so no load sits behind a branch.
__device__ __forceinline__ void dec_down_wave(const LayerDev &L, const Dims &D, bool ok, int e, int ti, int hrow,
                                              const uint32_t *__restrict__ hq, const float *__restrict__ hs,
                                              float *out) {
  const int lane = threadIdx.x & 63, C = D.f / kChunk;
  const ExpertLayout EL = expert_layout(D.d, D.f);
  const uint8_t *base = expert_base(L, ok ? e : 0);
  const __amdgpu_buffer_rsrc_t rn = wave_rsrc(base + EL.dn_nib, (uint32_t)(EL.dn_sc - EL.dn_nib));
  const __amdgpu_buffer_rsrc_t rs = wave_rsrc(base + EL.dn_sc, (uint32_t)(EL.bytes - EL.dn_sc));
  const int cl = lane < C ? lane : C - 1;
  // chunk_offset with one step per row: tile, then row r at r * C * 16 bytes
  const int tb = ti * kTileRows * (D.f / 2);
  u32x4 W[kTileRows];
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) W[r] = __builtin_amdgcn_raw_buffer_load_b128(rn, cl * 16, tb + r * C * 16, 0);
  const u32x4 Sv = __builtin_amdgcn_raw_buffer_load_b128(rs, (cl >> 1) * 16, ti * (D.f / kGroup) * 16, 0);
  uint32_t dg[kDigitWords];
  float dsc[2];
  load_digits(hq, hs, hrow, D.f, cl, dg, dsc);
  const uint4 S = make_uint4(Sv.x, Sv.y, Sv.z, Sv.w);
  float acc[kTileRows];
#pragma unroll
  for (int rr = 0; rr < kTileRows; ++rr) {
    const float a = fxp_chunk(make_uint4(W[rr].x, W[rr].y, W[rr].z, W[rr].w), dg, dsc, tile_scale(S, rr), 0.0f);
    acc[rr] = (ok && lane < C) ? a : 0.0f;
  }
  const float v = reduce8_rows(acc);
  if ((lane & 7) == 7) out[lane >> 3] = v;
}

__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(6))) void k_down_dec1(
    LayerDev L, Dims D, const uint32_t *__restrict__ hq, const float *__restrict__ hs, UnionDev U,
    const float *__restrict__ wslot, float *__restrict__ residual) {
  __shared__ float vb[16][kTileRows];
  __shared__ int ok_s[16];
  __shared__ float wsl_s[16];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ti = blockIdx.x;
  const int nu = clamp_nu(U.n_unique, D);
  const int slots = nu + D.n_shared;
  // the combine's inputs (slot gate weights, the residual tile) are fetched
  // by wave 0 before its weights, so they are in hand after the barrier
  float wl = 0.0f, rin = 0.0f;
  if (wave == 0) {
    wl = wslot[lane < kDecMaxSlots ? lane : kDecMaxSlots - 1];
    rin = residual[(size_t)ti * kTileRows + (lane & 7)];
  }
  if (wave < slots) {
    int e, p0, p1;
    const bool ok = resolve_slot(D, U, nu, wave, e, p0, p1) && p1 > p0;
    dec_down_wave(L, D, ok, e, ti, wave < nu ? p0 : D.T * D.k, hq, hs, vb[wave]);
    if (lane == 0) ok_s[wave] = ok;
  }
  if (wave == 0 && lane < kDecMaxSlots) wsl_s[lane] = wl;
  __syncthreads();
  if (wave == 0 && lane < kTileRows) {
    float out = rin;
    for (int sl = 0; sl < slots; ++sl) {
      if (!ok_s[sl]) continue;
      const float v = vb[sl][lane];
      out = sl < nu ? __builtin_fmaf(wsl_s[sl], v, out) : out + v;
    }
    residual[(size_t)ti * kTileRows + lane] = out;
  }
}


// Down + combine for 2-4 tokens when a down row is one step: a block per
// (token, 8-row output tile), one wave per top-k position of the token (the
// pair's h row, its expert from idx) plus the shared expert, the wave code of
// k_down_dec1; wave 0 then folds the outputs into the token's residual in
// pair order with the gate weights, then the shared expert's, as k_combine
// does.  Items are (tile, token) with the token fastest, the block ids
// remapped so each XCD takes one contiguous range: tokens of one tile that
// share an expert read its rows through one L2.
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(6))) void k_down_dec_tok(
    LayerDev L, Dims D, const uint32_t *__restrict__ hq, const float *__restrict__ hs, UnionDev U,
    const int32_t *__restrict__ idx, const float *__restrict__ w, float *__restrict__ residual, int n_items) {
  __shared__ float vb[kDecMaxSlots][kTileRows];
  __shared__ int ok_s[kDecMaxSlots], order_s[kDecMaxSlots], nsel_s;
  __shared__ float wsl_s[kDecMaxSlots];
  const int per = (int)gridDim.x / 8;
  const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (item >= n_items) return;  // block-uniform
  const int ti = item / D.T, t = item - ti * D.T;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int tk = D.T * D.k;
  const int nu = clamp_nu(U.n_unique, D);
  float rin = 0.0f;
  if (wave == 0) {
    // the token's pair positions ranked: the combine's order (experts
    // ascending), with each position's gate weight
    int p = 0x7FFFFFFF;
    float wv = 0.0f;
    if (nu > 0 && lane < D.k) {
      p = U.pair_of[(size_t)t * D.k + lane];
      if (p < 0 || p >= tk) p = 0x7FFFFFFF;
      wv = w[(size_t)t * D.k + lane];
    }
    int rank = 0, valid = 0;
    for (int i = 0; i < D.k; ++i) {
      const int q = __shfl(p, i, 64);
      rank += (q < p) || (q == p && i < lane);
      valid += q < tk;
    }
    if (lane < D.k && p < tk) order_s[rank] = lane;
    if (lane < kDecMaxSlots) wsl_s[lane] = wv;
    if (lane == 0) nsel_s = valid;
    rin = residual[(size_t)t * D.d + (size_t)ti * kTileRows + (lane & 7)];
  }
  if (wave < D.k + D.n_shared) {
    bool ok;
    int e, hrow;
    if (wave < D.k) {
      const int p = nu > 0 ? U.pair_of[(size_t)t * D.k + wave] : -1;
      e = idx[(size_t)t * D.k + wave];
      ok = p >= 0 && p < tk && e >= 0 && e < D.E;
      hrow = ok ? p : 0;
    } else {
      ok = true;
      e = D.E;
      hrow = tk + t;
    }
    // a position dropped by expert top-p loads nothing (the test is the same
    // for every lane of the wave)
    if (__builtin_amdgcn_readfirstlane((int)ok)) dec_down_wave(L, D, true, e, ti, hrow, hq, hs, vb[wave]);
    if (lane == 0) ok_s[wave] = ok;
  }
  __syncthreads();
  if (wave == 0 && lane < kTileRows) {
    float out = rin;
    const int n = nsel_s;
    for (int r = 0; r < n; ++r) {
      const int j = order_s[r];
      if (ok_s[j]) out = __builtin_fmaf(wsl_s[j], vb[j][lane], out);
    }
    if (D.n_shared) out = out + vb[D.k][lane];
    residual[(size_t)t * D.d + (size_t)ti * kTileRows + lane] = out;
  }
}

// Down projection and combine of the fp32 one-token pair: a block per 8-row
// output tile, one wave per slot (up to kDecMaxSlots), few enough registers
// that a decode call's blocks are resident together.  Per (row, slot) the
// operations are those of k_down_wide (the lane's chunks in order,
// fma(scale, chunk_dot, acc), the fixed 8-row tree), and the combine adds
// the routed experts in ascending pair order with their gate weights, then
// the shared expert, as combine_tile does: the bits are those of the fused
// k_down_wide.  h rows come in the pair's interleaved layout (h_ilv), with
// the two half-chunk sums the gate/up kernel formed in neg8_sum's order
// (hsum), so chunk_dot can run a word's 8 columns at a time for all 8 rows
// with only those columns' activations in registers.
// One wave of the fp32 one-token down kernels: the 8 rows of output tile ti
// of expert e (when ok) against h row hrow (the pair's interleaved layout,
// with its chunk sums in hsum), reduced by the fixed tree into out[0..8).
__device__ __forceinline__ void f32_down_wave(const LayerDev &L, const Dims &D, bool ok, int e, int ti, int hrow,
                                              const float *__restrict__ h, const float *__restrict__ hsum,
                                              float *out) {
  const int lane = threadIdx.x & 63, C = D.f / kChunk;
  const ExpertLayout EL = expert_layout(D.d, D.f);
  // buffer loads: the lane's offset in a VGPR, the rest in the scalar
  // offset; a lane past the row end reads a valid chunk (the row's last)
  // and keeps its sums unchanged
  const uint8_t *base = expert_base(L, ok ? e : 0);
  const __amdgpu_buffer_rsrc_t rn = wave_rsrc(base + EL.dn_nib, (uint32_t)(EL.dn_sc - EL.dn_nib));
  const __amdgpu_buffer_rsrc_t rs = wave_rsrc(base + EL.dn_sc, (uint32_t)(EL.bytes - EL.dn_sc));
  const __amdgpu_buffer_rsrc_t rh = wave_rsrc(h + (size_t)hrow * D.f, (uint32_t)D.f * 4u);
  const __amdgpu_buffer_rsrc_t rq = wave_rsrc(hsum + (size_t)hrow * (D.f / 16), (uint32_t)D.f / 4u);
  float acc[kTileRows];
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) acc[r] = 0.0f;
  for (int j = 0; 64 * j < C; ++j) {
    const int width = C - 64 * j < 64 ? C - 64 * j : 64;
    const bool live = lane < width;
    const int cl = live ? lane : width - 1;
    const int tb = ti * kTileRows * (D.f / 2) + j * (kTileRows * 64 * 16);
    uint4 W[kTileRows];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rn, cl * 16, tb + r * width * 16, 0);
      W[r] = make_uint4(t.x, t.y, t.z, t.w);
    }
    const u32x4 Sv =
        __builtin_amdgcn_raw_buffer_load_b128(rs, (cl >> 1) * 16, (ti * (D.f / kGroup) + 32 * j) * 16, 0);
    const uint4 S = make_uint4(Sv.x, Sv.y, Sv.z, Sv.w);
    // -8 sum of the chunk's 32 activations: the two halves in order
    const u32x2 hq2 = __builtin_amdgcn_raw_buffer_load_b64(rq, cl * 8, 64 * j * 8, 0);
    const float nsx = -8.0f * (bits_f(hq2[0]) + bits_f(hq2[1]));
    float alo[kTileRows], ahi[kTileRows];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      alo[r] = nsx;
      ahi[r] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // (elements by index: hipcc turns __builtin_bit_cast of a vector
      // element .y/.z/.w into element 0)
      const u32x4 ta = __builtin_amdgcn_raw_buffer_load_b128(rh, cl * 16, ((2 * i) * C + 64 * j) * 16, 0);
      const u32x4 tb2 = __builtin_amdgcn_raw_buffer_load_b128(rh, cl * 16, ((2 * i + 1) * C + 64 * j) * 16, 0);
      const float4 xa = make_float4(bits_f(ta[0]), bits_f(ta[1]), bits_f(ta[2]), bits_f(ta[3]));
      const float4 xb = make_float4(bits_f(tb2[0]), bits_f(tb2[1]), bits_f(tb2[2]), bits_f(tb2[3]));
#pragma unroll
      for (int r = 0; r < kTileRows; ++r) {
        const uint32_t wi = (i == 0 ? W[r].x : i == 1 ? W[r].y : i == 2 ? W[r].z : W[r].w) ^ 0x88888888u;
        uint32_t lo = wi & 0x0F0F0F0Fu, hi = wi & 0xF0F0F0F0u;
        asm("" : "+v"(lo), "+v"(hi));
        alo[r] = __builtin_fmaf((float)(lo & 0xFFu), xa.x, alo[r]);
        alo[r] = __builtin_fmaf((float)((lo >> 8) & 0xFFu), xa.z, alo[r]);
        alo[r] = __builtin_fmaf((float)((lo >> 16) & 0xFFu), xb.x, alo[r]);
        alo[r] = __builtin_fmaf((float)(lo >> 24), xb.z, alo[r]);
        ahi[r] = __builtin_fmaf((float)(hi & 0xFFu), xa.y, ahi[r]);
        ahi[r] = __builtin_fmaf((float)((hi >> 8) & 0xFFu), xa.w, ahi[r]);
        ahi[r] = __builtin_fmaf((float)((hi >> 16) & 0xFFu), xb.y, ahi[r]);
        ahi[r] = __builtin_fmaf((float)(hi >> 24), xb.w, ahi[r]);
      }
      // the word's sums are due here: one word's masks and activations
      // live at a time
#pragma unroll
      for (int r = 0; r < kTileRows; ++r) asm volatile("" : "+v"(alo[r]), "+v"(ahi[r]));
    }
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      const float a = __builtin_fmaf(tile_scale(S, r), __builtin_fmaf(ahi[r], 0.0625f, alo[r]), acc[r]);
      acc[r] = live ? a : acc[r];
    }
  }
  const float v = reduce8_rows(acc);
  if ((lane & 7) == 7) out[lane >> 3] = v;
}

__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(7))) void k_down_f32_dec(
    LayerDev L, Dims D, const float *__restrict__ h, const float *__restrict__ hsum, UnionDev U,
    const float *__restrict__ w, float *__restrict__ residual) {
  __shared__ float vb[kDecMaxSlots][kTileRows];
  __shared__ int ok_s[kDecMaxSlots];
  __shared__ float wsl_s[kDecMaxSlots];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ti = blockIdx.x;
  const int nu = clamp_nu(U.n_unique, D);
  const int slots = nu + D.n_shared;
  float rin = 0.0f;
  if (wave == 0 && lane < kTileRows) rin = residual[(size_t)ti * kTileRows + lane];
  if (wave < slots) {
    int e, p0, p1;
    const bool ok = resolve_slot(D, U, nu, wave, e, p0, p1) && p1 > p0;
    if (lane == 0) {
      float g = 1.0f;
      if (wave < nu) {
        int js = U.pair_slot[p0];
        js = js < 0 ? 0 : (js >= D.k ? D.k - 1 : js);  // caller-supplied lists stay in bounds
        g = w[js];
      }
      wsl_s[wave] = g;
      ok_s[wave] = ok;
    }
    f32_down_wave(L, D, ok, e, ti, wave < nu ? p0 : D.T * D.k, h, hsum, vb[wave]);
  }
  __syncthreads();
  if (wave == 0 && lane < kTileRows) {
    float out = rin;
    for (int sl = 0; sl < nu; ++sl)
      if (ok_s[sl]) out = __builtin_fmaf(wsl_s[sl], vb[sl][lane], out);
    if (D.n_shared && ok_s[nu]) out = out + vb[nu][lane];
    residual[(size_t)ti * kTileRows + lane] = out;
  }
}

// The fp32 pair for 2-4 tokens: down + combine per (token, 8-row output
// tile), one wave per top-k position of the token (the pair's h row, its
// expert from idx) plus the shared expert, the wave code of k_down_f32_dec;
// wave 0 folds into the token's residual in pair order as k_combine does.
// Items and block ids as in k_down_dec_tok.
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(7))) void k_down_f32_tok(
    LayerDev L, Dims D, const float *__restrict__ h, const float *__restrict__ hsum, UnionDev U,
    const int32_t *__restrict__ idx, const float *__restrict__ w, float *__restrict__ residual, int n_items) {
  __shared__ float vb[kDecMaxSlots][kTileRows];
  __shared__ int ok_s[kDecMaxSlots], order_s[kDecMaxSlots], nsel_s;
  __shared__ float wsl_s[kDecMaxSlots];
  const int per = (int)gridDim.x / 8;
  const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (item >= n_items) return;  // block-uniform
  const int ti = item / D.T, t = item - ti * D.T;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int tk = D.T * D.k;
  const int nu = clamp_nu(U.n_unique, D);
  float rin = 0.0f;
  if (wave == 0) {
    int p = 0x7FFFFFFF;
    float wv = 0.0f;
    if (nu > 0 && lane < D.k) {
      p = U.pair_of[(size_t)t * D.k + lane];
      if (p < 0 || p >= tk) p = 0x7FFFFFFF;
      wv = w[(size_t)t * D.k + lane];
    }
    int rank = 0, valid = 0;
    for (int i = 0; i < D.k; ++i) {
      const int q = __shfl(p, i, 64);
      rank += (q < p) || (q == p && i < lane);
      valid += q < tk;
    }
    if (lane < D.k && p < tk) order_s[rank] = lane;
    if (lane < kDecMaxSlots) wsl_s[lane] = wv;
    if (lane == 0) nsel_s = valid;
    rin = residual[(size_t)t * D.d + (size_t)ti * kTileRows + (lane & 7)];
  }
  if (wave < D.k + D.n_shared) {
    bool ok;
    int e, hrow;
    if (wave < D.k) {
      const int p = nu > 0 ? U.pair_of[(size_t)t * D.k + wave] : -1;
      e = idx[(size_t)t * D.k + wave];
      ok = p >= 0 && p < tk && e >= 0 && e < D.E;
      hrow = ok ? p : 0;
    } else {
      ok = true;
      e = D.E;
      hrow = tk + t;
    }
    // a position dropped by expert top-p loads nothing
    if (__builtin_amdgcn_readfirstlane((int)ok)) f32_down_wave(L, D, true, e, ti, hrow, h, hsum, vb[wave]);
    if (lane == 0) ok_s[wave] = ok;
  }
  __syncthreads();
  if (wave == 0 && lane < kTileRows) {
    float out = rin;
    const int n = nsel_s;
    for (int r = 0; r < n; ++r) {
      const int j = order_s[r];
      if (ok_s[j]) out = __builtin_fmaf(wsl_s[j], vb[j][lane], out);
    }
    if (D.n_shared) out = out + vb[D.k][lane];
    residual[(size_t)t * D.d + (size_t)ti * kTileRows + lane] = out;
  }
}

// ------------------------------------------------------- int8 container
// Experts stored as int8 gs64 (one two's-complement byte per weight, the
// canonical blob layout [gate q][gate s][up q][up s][down q][down s], rows
// row-major): the pages keep the MTP head in int8 because int4 lost too much
// precision there ([P] lessons on record; [D] §4 highlight 2).  One wave per
// output row of one unique-expert slot; a lane takes 16-column chunks (one
// 16-byte load) lane, lane + 64, ...; each byte is flipped to offset binary
// n = q + 128 (XOR 0x80) and converted, and -128 * (sum of the chunk's
// activations) starts the chunk's sum, so sum n x - 128 sum x = sum q x;
// times the group scale, accumulated in fp32; the wave's partials are summed
// by the fixed tree of wave_sum.  The slot's tokens are taken kI8Tok at a
// time, each chunk's weights loaded once for all of them (the batch-union
// read of [A] §2); per token the operations do not depend on the others, so
// a token's bits are those of the token alone.
constexpr int kI8Tok = 4;

// Sum over 16 columns of (n_i - 128) x_i for the 16 bytes of w and x[0..15].
__device__ __forceinline__ float chunk_dot_i8(const uint4 &w, const float4 (&xv)[4]) {
  const uint32_t ws[4] = {w.x ^ 0x80808080u, w.y ^ 0x80808080u, w.z ^ 0x80808080u, w.w ^ 0x80808080u};
  float sx = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) sx = sx + ((xv[i].x + xv[i].y) + (xv[i].z + xv[i].w));
  float acc = -128.0f * sx;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = __builtin_fmaf((float)(ws[i] & 0xFFu), xv[i].x, acc);
    acc = __builtin_fmaf((float)((ws[i] >> 8) & 0xFFu), xv[i].y, acc);
    acc = __builtin_fmaf((float)((ws[i] >> 16) & 0xFFu), xv[i].z, acc);
    acc = __builtin_fmaf((float)(ws[i] >> 24), xv[i].w, acc);
  }
  return acc;
}

__device__ __forceinline__ float half_at(const uint8_t *p, size_t i) {
  return (float)__builtin_bit_cast(_Float16, *(const uint16_t *)(p + 2 * i));
}

// Slot s of a one-token call: expert, output row and activation row; false
// for a slot that holds nothing.
__device__ __forceinline__ bool slot_i8(const Dims &D, const UnionDev &U, int s, int &e, int &orow) {
  const int nu = clamp_nu(U.n_unique, D);
  if (s > nu || (s == nu && !D.n_shared)) return false;
  int p0, p1;
  if (!resolve_slot(D, U, nu, s, e, p0, p1) || p1 <= p0) return false;
  orow = s < nu ? p0 : D.T * D.k;
  return true;
}

// One token: h[orow][j] = SiLU(gate_j . x) * (up_j . x); grid (f/4, slots),
// 4 waves a block (the per-token operations of k_gateup_i8, without the
// token loop).
__global__ __launch_bounds__(256) void k_gateup_i8_one(LayerDev L, Dims D, const float *__restrict__ x, UnionDev U,
                                                   float *__restrict__ h) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + wave;
  int e, orow;
  if (j >= D.f || !slot_i8(D, U, blockIdx.y, e, orow)) return;
  const size_t w = (size_t)D.d * D.f, ns = w / kGroup * 2;
  const uint8_t *base = expert_base(L, e);
  const uint8_t *gq = base + (size_t)j * D.d, *uq = base + w + ns + (size_t)j * D.d;
  const uint8_t *gs = base + w + (size_t)j * (D.d / kGroup) * 2, *us = base + 2 * w + ns + (size_t)j * (D.d / kGroup) * 2;
  float ag = 0.0f, au = 0.0f;
  for (int c = lane; c < D.d / 16; c += 64) {
    const uint4 wg = *(const uint4 *)(gq + 16 * (size_t)c), wu = *(const uint4 *)(uq + 16 * (size_t)c);
    float4 xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = *(const float4 *)(x + 16 * (size_t)c + 4 * i);
    ag = __builtin_fmaf(half_at(gs, c >> 2), chunk_dot_i8(wg, xv), ag);
    au = __builtin_fmaf(half_at(us, c >> 2), chunk_dot_i8(wu, xv), au);
  }
  const float g = wave_sum(ag), u = wave_sum(au);
  if (lane == 0) h[(size_t)orow * D.f + j] = silu_f(g) * u;
}

// One token: y[orow][r] = down_r . h[orow]; grid (d/4, slots), 4 waves a block.
__global__ __launch_bounds__(256) void k_down_i8_one(LayerDev L, Dims D, const float *__restrict__ h, UnionDev U,
                                                 float *__restrict__ y) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  int e, orow;
  if (r >= D.d || !slot_i8(D, U, blockIdx.y, e, orow)) return;
  const size_t w = (size_t)D.d * D.f, ns = w / kGroup * 2;
  const uint8_t *base = expert_base(L, e) + 2 * (w + ns);
  const uint8_t *dq = base + (size_t)r * D.f, *ds = base + w + (size_t)r * (D.f / kGroup) * 2;
  const float *hr = h + (size_t)orow * D.f;
  float acc = 0.0f;
  for (int c = lane; c < D.f / 16; c += 64) {
    const uint4 wd = *(const uint4 *)(dq + 16 * (size_t)c);
    float4 hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = *(const float4 *)(hr + 16 * (size_t)c + 4 * i);
    acc = __builtin_fmaf(half_at(ds, c >> 2), chunk_dot_i8(wd, hv), acc);
  }
  const float v = wave_sum(acc);
  if (lane == 0) y[(size_t)orow * D.d + r] = v;
}

// The one-token int8 kernels of a decode call.  Per row they perform the
// operations of k_gateup_i8_one and k_down_i8_one (lane l takes chunks l,
// l + 64, ... in order, fma(scale, chunk_dot_i8, acc), the wave_sum tree), so
// the bits are those of the batched int8 kernels; what changes is how many
// loads a wave has in flight.  Gate/up: a wave per h output issues all NI
// chunks of its gate and up rows before the arithmetic (a lane past the row
// end loads the row's last chunk and adds nothing).  Down: a block per
// kI8Rows output rows (8: every block reads all slots' h rows, so taller
// tiles read h fewer times), a wave per slot issuing its NI chunks of every
// row at once; wave 0 then folds the slot outputs into the residual in the
// order of k_combine (routed experts in pair order, each times its gate
// weight, then the shared expert).
constexpr int kI8Rows = 8;
template <int NI, bool PAIRS>
__global__ __launch_bounds__(256) void k_gateup_i8_dec(LayerDev L, Dims D, const float *__restrict__ x, UnionDev U,
                                                       float *__restrict__ h, const int32_t *__restrict__ idx,
                                                       int n_items) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int j, e, orow;
  if (PAIRS) {
    // 2-16 tokens: items (4 h outputs, pair) with the pair fastest, spread
    // over the XCDs in contiguous ranges as in k_gateup_pairs; the pair's
    // token and expert as there (every lane resolves the same pair)
    const int per = (int)gridDim.x / 8;
    const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (item >= n_items) return;
    const int tk = D.T * D.k, P = tk + D.T * D.n_shared;
    const int jg = item / P, p = item - jg * P;
    j = jg * 4 + wave;
    if (j >= D.f) return;
    int t = 0;
    e = -1;
    if (p < tk) {
      const int nu = clamp_nu(U.n_unique, D);
      int np = U.offsets[nu];
      np = np < 0 ? 0 : (np > tk ? tk : np);
      t = U.pair_token[p];
      const int js = U.pair_slot[p];
      if (p < np && t >= 0 && t < D.T && js >= 0 && js < D.k) {
        e = idx[(size_t)t * D.k + js];
        if (e < 0 || e >= D.E) e = -1;
      }
    } else {
      t = p - tk;
      e = D.E;
    }
    if (e < 0) return;
    orow = p;
    x += (size_t)t * D.d;
  } else {
    j = blockIdx.x * 4 + wave;
    if (j >= D.f || !slot_i8(D, U, blockIdx.y, e, orow)) return;
  }
  const size_t w = (size_t)D.d * D.f, ns = w / kGroup * 2;
  const uint8_t *base = expert_base(L, e);
  const uint8_t *gq = base + (size_t)j * D.d, *uq = base + w + ns + (size_t)j * D.d;
  const uint8_t *gs = base + w + (size_t)j * (D.d / kGroup) * 2, *us = base + 2 * w + ns + (size_t)j * (D.d / kGroup) * 2;
  const int C = D.d / 16;
  uint4 Wg[NI], Wu[NI];
  float sg[NI], su[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = lane + 64 * i, cl = c < C ? c : C - 1;
    Wg[i] = *(const uint4 *)(gq + 16 * (size_t)cl);
    Wu[i] = *(const uint4 *)(uq + 16 * (size_t)cl);
    sg[i] = half_at(gs, cl >> 2);
    su[i] = half_at(us, cl >> 2);
  }
  float ag = 0.0f, au = 0.0f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = lane + 64 * i;
    if (c < C) {
      float4 xv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) xv[k] = *(const float4 *)(x + 16 * (size_t)c + 4 * k);
      ag = __builtin_fmaf(sg[i], chunk_dot_i8(Wg[i], xv), ag);
      au = __builtin_fmaf(su[i], chunk_dot_i8(Wu[i], xv), au);
    }
  }
  const float g = wave_sum(ag), u = wave_sum(au);
  if (lane == 0) h[(size_t)orow * D.f + j] = silu_f(g) * u;
}

// One wave of the int8 one-token down kernels: rows r0..r0+7 of expert e's
// down matrix against h row hrow, lane l taking chunks l, l + 64, ... in
// order, fma(scale, chunk_dot_i8, acc), the wave_sum tree; into out[0..8).
template <int NI>
__device__ __forceinline__ void i8_down_wave(const LayerDev &L, const Dims &D, int e, int r0, int hrow,
                                             const float *__restrict__ h, float *out) {
  const int lane = threadIdx.x & 63;
  const size_t wsz = (size_t)D.d * D.f, ns = wsz / kGroup * 2;
  const uint8_t *dq = expert_base(L, e) + 2 * (wsz + ns);
  const uint8_t *ds = dq + wsz;
  const float *hr = h + (size_t)hrow * D.f;
  const int C = D.f / 16;
  uint4 W[kI8Rows][NI];
  float sc[kI8Rows][NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = lane + 64 * i, cl = c < C ? c : C - 1;
#pragma unroll
    for (int r = 0; r < kI8Rows; ++r) {
      W[r][i] = *(const uint4 *)(dq + (size_t)(r0 + r) * D.f + 16 * (size_t)cl);
      sc[r][i] = half_at(ds + (size_t)(r0 + r) * (D.f / kGroup) * 2, cl >> 2);
    }
  }
  float acc[kI8Rows];
#pragma unroll
  for (int r = 0; r < kI8Rows; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = lane + 64 * i;
    if (c < C) {
      float4 hv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) hv[k] = *(const float4 *)(hr + 16 * (size_t)c + 4 * k);
#pragma unroll
      for (int r = 0; r < kI8Rows; ++r) acc[r] = __builtin_fmaf(sc[r][i], chunk_dot_i8(W[r][i], hv), acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < kI8Rows; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == 0) out[r] = v;
  }
}

template <int NI>
__global__ __launch_bounds__(64 * kDecMaxSlots) void k_down_i8_dec(LayerDev L, Dims D, const float *__restrict__ h,
                                                                UnionDev U, const float *__restrict__ w,
                                                                float *__restrict__ residual) {
  __shared__ float vb[kDecMaxSlots][kI8Rows];
  __shared__ int ok_s[kDecMaxSlots];
  __shared__ float wsl_s[kDecMaxSlots];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = blockIdx.x * kI8Rows;
  const int nu = clamp_nu(U.n_unique, D);
  const int slots = nu + D.n_shared;
  float rin = 0.0f;
  if (wave == 0 && lane < kI8Rows) rin = residual[r0 + lane];
  if (wave < slots) {
    int e, p0, p1;
    const bool ok = resolve_slot(D, U, nu, wave, e, p0, p1) && p1 > p0;
    if (lane == 0) {
      float g = 1.0f;
      if (wave < nu) {
        int js = U.pair_slot[p0];
        js = js < 0 ? 0 : (js >= D.k ? D.k - 1 : js);  // caller-supplied lists stay in bounds
        g = w[js];
      }
      wsl_s[wave] = g;
      ok_s[wave] = ok;
    }
    i8_down_wave<NI>(L, D, ok ? e : 0, r0, wave < nu ? p0 : D.T * D.k, h, vb[wave]);
  }
  __syncthreads();
  if (wave == 0 && lane < kI8Rows) {
    float out = rin;
    for (int sl = 0; sl < nu; ++sl)
      if (ok_s[sl]) out = __builtin_fmaf(wsl_s[sl], vb[sl][lane], out);
    if (D.n_shared && ok_s[nu]) out = out + vb[nu][lane];
    residual[r0 + lane] = out;
  }
}

// The int8 pair for 2-16 tokens: down + combine per (token, 8 output rows),
// one wave per top-k position of the token (the pair's h row, its expert from
// idx) plus the shared expert, the wave code of k_down_i8_dec; wave 0 folds
// into the token's residual in pair order as k_combine does.  Items and
// block ids as in k_down_dec_tok.
template <int NI>
__global__ __launch_bounds__(64 * kDecMaxSlots) void k_down_i8_tok(LayerDev L, Dims D, const float *__restrict__ h,
                                                                UnionDev U, const int32_t *__restrict__ idx,
                                                                const float *__restrict__ w,
                                                                float *__restrict__ residual, int n_items) {
  __shared__ float vb[kDecMaxSlots][kI8Rows];
  __shared__ int ok_s[kDecMaxSlots], order_s[kDecMaxSlots], nsel_s;
  __shared__ float wsl_s[kDecMaxSlots];
  const int per = (int)gridDim.x / 8;
  const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (item >= n_items) return;  // block-uniform
  const int rb = item / D.T, t = item - rb * D.T, r0 = rb * kI8Rows;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int tk = D.T * D.k;
  const int nu = clamp_nu(U.n_unique, D);
  float rin = 0.0f;
  if (wave == 0) {
    int p = 0x7FFFFFFF;
    float wv = 0.0f;
    if (nu > 0 && lane < D.k) {
      p = U.pair_of[(size_t)t * D.k + lane];
      if (p < 0 || p >= tk) p = 0x7FFFFFFF;
      wv = w[(size_t)t * D.k + lane];
    }
    int rank = 0, valid = 0;
    for (int i = 0; i < D.k; ++i) {
      const int q = __shfl(p, i, 64);
      rank += (q < p) || (q == p && i < lane);
      valid += q < tk;
    }
    if (lane < D.k && p < tk) order_s[rank] = lane;
    if (lane < kDecMaxSlots) wsl_s[lane] = wv;
    if (lane == 0) nsel_s = valid;
    rin = residual[(size_t)t * D.d + r0 + (lane & 7)];
  }
  if (wave < D.k + D.n_shared) {
    bool ok;
    int e, hrow;
    if (wave < D.k) {
      const int p = nu > 0 ? U.pair_of[(size_t)t * D.k + wave] : -1;
      e = idx[(size_t)t * D.k + wave];
      ok = p >= 0 && p < tk && e >= 0 && e < D.E;
      hrow = ok ? p : 0;
    } else {
      ok = true;
      e = D.E;
      hrow = tk + t;
    }
    // a position dropped by expert top-p loads nothing
    if (__builtin_amdgcn_readfirstlane((int)ok)) i8_down_wave<NI>(L, D, e, r0, hrow, h, vb[wave]);
    if (lane == 0) ok_s[wave] = ok;
  }
  __syncthreads();
  if (wave == 0 && lane < kI8Rows) {
    float out = rin;
    const int n = nsel_s;
    for (int r = 0; r < n; ++r) {
      const int jj = order_s[r];
      if (ok_s[jj]) out = __builtin_fmaf(wsl_s[jj], vb[jj][lane], out);
    }
    if (D.n_shared) out = out + vb[D.k][lane];
    residual[(size_t)t * D.d + r0 + lane] = out;
  }
}

// h[orow][j] = SiLU(gate_j . x_t) * (up_j . x_t) for every pair (t, orow) of
// slot blockIdx.y; grid (f/4, slots), 4 waves a block.
__global__ __launch_bounds__(256) void k_gateup_i8(LayerDev L, Dims D, const float *__restrict__ x, UnionDev U,
                                                   float *__restrict__ h) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + wave, s = blockIdx.y;
  const int nu = clamp_nu(U.n_unique, D);
  int e, p0, p1;
  if (j >= D.f || s > nu || (s == nu && !D.n_shared) || !resolve_slot(D, U, nu, s, e, p0, p1)) return;
  const size_t w = (size_t)D.d * D.f, ns = w / kGroup * 2;
  const uint8_t *base = expert_base(L, e);
  const uint8_t *gq = base + (size_t)j * D.d, *uq = base + w + ns + (size_t)j * D.d;
  const uint8_t *gs = base + w + (size_t)j * (D.d / kGroup) * 2, *us = base + 2 * w + ns + (size_t)j * (D.d / kGroup) * 2;
  for (int pg = p0; pg < p1; pg += kI8Tok) {
    const int mc = min(kI8Tok, p1 - pg);
    int tm[kI8Tok], om[kI8Tok];
    float ag[kI8Tok], au[kI8Tok];
#pragma unroll
    for (int m = 0; m < kI8Tok; ++m) {
      tm[m] = 0;
      om[m] = -1;
      if (m < mc) slot_token(D, U, nu, s, pg + m, tm[m], om[m]);
      ag[m] = 0.0f;
      au[m] = 0.0f;
    }
    for (int c = lane; c < D.d / 16; c += 64) {
      const uint4 wg = *(const uint4 *)(gq + 16 * (size_t)c), wu = *(const uint4 *)(uq + 16 * (size_t)c);
      const float sg = half_at(gs, c >> 2), su = half_at(us, c >> 2);
#pragma unroll
      for (int m = 0; m < kI8Tok; ++m)
        if (m < mc) {
          float4 xv[4];
          const float *xr = x + (size_t)tm[m] * D.d;
#pragma unroll
          for (int i = 0; i < 4; ++i) xv[i] = *(const float4 *)(xr + 16 * (size_t)c + 4 * i);
          ag[m] = __builtin_fmaf(sg, chunk_dot_i8(wg, xv), ag[m]);
          au[m] = __builtin_fmaf(su, chunk_dot_i8(wu, xv), au[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < kI8Tok; ++m)
      if (m < mc) {
        const float g = wave_sum(ag[m]), u = wave_sum(au[m]);
        if (lane == 0 && om[m] >= 0) h[(size_t)om[m] * D.f + j] = silu_f(g) * u;
      }
  }
}

// y[orow][r] = down_r . h[orow] for every pair of slot blockIdx.y; grid
// (d/4, slots), 4 waves a block.
__global__ __launch_bounds__(256) void k_down_i8(LayerDev L, Dims D, const float *__restrict__ h, UnionDev U,
                                                 float *__restrict__ y) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave, s = blockIdx.y;
  const int nu = clamp_nu(U.n_unique, D);
  int e, p0, p1;
  if (r >= D.d || s > nu || (s == nu && !D.n_shared) || !resolve_slot(D, U, nu, s, e, p0, p1)) return;
  const size_t w = (size_t)D.d * D.f, ns = w / kGroup * 2;
  const uint8_t *base = expert_base(L, e) + 2 * (w + ns);
  const uint8_t *dq = base + (size_t)r * D.f, *ds = base + w + (size_t)r * (D.f / kGroup) * 2;
  for (int pg = p0; pg < p1; pg += kI8Tok) {
    const int mc = min(kI8Tok, p1 - pg);
    int om[kI8Tok];
    float acc[kI8Tok];
#pragma unroll
    for (int m = 0; m < kI8Tok; ++m) {
      int t = 0;
      om[m] = -1;
      if (m < mc) slot_token(D, U, nu, s, pg + m, t, om[m]);
      acc[m] = 0.0f;
    }
    for (int c = lane; c < D.f / 16; c += 64) {
      const uint4 wd = *(const uint4 *)(dq + 16 * (size_t)c);
      const float sd = half_at(ds, c >> 2);
#pragma unroll
      for (int m = 0; m < kI8Tok; ++m)
        if (m < mc && om[m] >= 0) {
          float4 hv[4];
          const float *hr = h + (size_t)om[m] * D.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) hv[i] = *(const float4 *)(hr + 16 * (size_t)c + 4 * i);
          acc[m] = __builtin_fmaf(sd, chunk_dot_i8(wd, hv), acc[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < kI8Tok; ++m)
      if (m < mc) {
        const float v = wave_sum(acc[m]);
        if (lane == 0 && om[m] >= 0) y[(size_t)om[m] * D.d + r] = v;
      }
  }
}

// ------------------------------------------------- narrow shapes (K < 2048)
// Rows shorter than 64 chunks: LPR lanes per row (a power of two >= K/32,
// one chunk per lane), 64/LPR rows side by side in a wave, one wave per
// (slot, 8-row tile).  Same arithmetic per chunk; reductions by a fixed
// butterfly within LPR lanes.

template <int LPR>
struct NarrowShape {
  static constexpr int RG = 64 / LPR;                    // row groups per wave
  static constexpr int RPG = (kTileRows + RG - 1) / RG;  // rows per lane
};

template <int LPR, int MT>
__device__ __forceinline__ void narrow_tile(const uint8_t *__restrict__ nib, const uint8_t *__restrict__ sc, int tile,
                                            int K, const float *__restrict__ xbase, size_t xstride,
                                            const int (&xrow)[MT], int mcount,
                                            float (&acc)[MT][NarrowShape<LPR>::RPG]) {
  using NS = NarrowShape<LPR>;
  const int lane = threadIdx.x & 63;
  const int q = lane % LPR, gr = lane / LPR;
  const int C = K / kChunk, G = K / kGroup;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < NS::RPG; ++i) acc[m][i] = 0.0f;
  if (q >= C) return;
  const uint4 S = *(const uint4 *)(sc + ((size_t)tile * G + (q >> 1)) * 16);
#pragma unroll
  for (int i = 0; i < NS::RPG; ++i) {
    const int r = gr + NS::RG * i;
    if (r < kTileRows) {
      const uint4 Wr = *(const uint4 *)(nib + chunk_offset(tile, K, q, r));
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < mcount) {
          float4 xv[8];
          const float4 *src = (const float4 *)(xbase + (size_t)xrow[m] * xstride + (size_t)kChunk * q);
#pragma unroll
          for (int v = 0; v < 8; ++v) xv[v] = src[v];
          acc[m][i] = __builtin_fmaf(tile_scale(S, r), chunk_dot(Wr, xv, neg8_sum(xv)), acc[m][i]);
        }
    }
  }
}

template <int LPR>
__device__ __forceinline__ void narrow_reduce(const float *acc, float *rows) {
  using NS = NarrowShape<LPR>;
  const int lane = threadIdx.x & 63;
  const int q = lane % LPR, gr = lane / LPR;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < NS::RPG; ++i) {
    const float v = group_sum(acc[i], LPR);
    const int r = gr + NS::RG * i;
    if (q == 0 && r < kTileRows) rows[r] = v;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int LPR, int MT>
__global__ __launch_bounds__(256) void k_gateup_narrow(LayerDev L, Dims D, const float *__restrict__ x, UnionDev U,
                                                       float *__restrict__ h, float *__restrict__ gdbg,
                                                       float *__restrict__ udbg) {
  using NS = NarrowShape<LPR>;
  __shared__ float rows_lds[4][kTileRows];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tiles = D.f / 4;
  const int nu = clamp_nu(U.n_unique, D);
  const int active = (nu + D.n_shared) * tiles;
  const ExpertLayout EL = expert_layout(D.d, D.f);
  for (int item = blockIdx.x * 4 + wave; item < active; item += gridDim.x * 4) {
    const int s = item / tiles, ti = item - s * tiles;
    int e, p0, p1;
    if (!resolve_slot(D, U, nu, s, e, p0, p1)) continue;
    const uint8_t *base = expert_base(L, e);
    for (int pg = p0; pg < p1; pg += MT) {
      const int mcount = min(MT, p1 - pg);
      int xrow[MT], orows[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        int t = 0, orow = -1;
        if (m < mcount) slot_token(D, U, nu, s, pg + m, t, orow);
        xrow[m] = t;
        orows[m] = orow;
      }
      float acc[MT][NS::RPG];
      narrow_tile<LPR, MT>(base + EL.gu_nib, base + EL.gu_sc, ti, D.d, x, (size_t)D.d, xrow, mcount, acc);
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < mcount) {
          narrow_reduce<LPR>(acc[m], rows_lds[wave]);
          if (lane < 4 && orows[m] >= 0) {
            const float g = rows_lds[wave][lane], u = rows_lds[wave][lane + 4];
            const size_t o = (size_t)orows[m] * D.f + (size_t)ti * 4 + lane;
            h[o] = silu_f(g) * u;
            if (gdbg) {
              gdbg[o] = g;
              udbg[o] = u;
            }
          }
        }
    }
  }
}

template <int LPR, int MT>
__global__ __launch_bounds__(256) void k_down_narrow(LayerDev L, Dims D, const float *__restrict__ h, UnionDev U,
                                                     float *__restrict__ y) {
  using NS = NarrowShape<LPR>;
  __shared__ float rows_lds[4][kTileRows];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tiles = D.d / kTileRows;
  const int nu = clamp_nu(U.n_unique, D);
  const int active = (nu + D.n_shared) * tiles;
  const ExpertLayout EL = expert_layout(D.d, D.f);
  for (int item = blockIdx.x * 4 + wave; item < active; item += gridDim.x * 4) {
    const int s = item / tiles, ti = item - s * tiles;
    int e, p0, p1;
    if (!resolve_slot(D, U, nu, s, e, p0, p1)) continue;
    const uint8_t *base = expert_base(L, e);
    for (int pg = p0; pg < p1; pg += MT) {
      const int mcount = min(MT, p1 - pg);
      int orows[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) orows[m] = m < mcount ? ((s < nu) ? pg + m : D.T * D.k + pg + m) : 0;
      float acc[MT][NS::RPG];
      narrow_tile<LPR, MT>(base + EL.dn_nib, base + EL.dn_sc, ti, D.f, h, (size_t)D.f, orows, mcount, acc);
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < mcount) {
          narrow_reduce<LPR>(acc[m], rows_lds[wave]);
          if (lane < kTileRows) y[(size_t)orows[m] * D.d + (size_t)ti * kTileRows + lane] = rows_lds[wave][lane];
        }
    }
  }
}

// Down + combine for one token on the narrow shapes (f < 2048): a block per
// 8-row output tile, one wave per slot (up to kDecMaxSlots) with the
// operations of k_down_narrow (narrow_tile, narrow_reduce) on the slot's h
// row; wave 0 folds the slots' rows into the residual as k_combine does
// (routed slots in pair order, which for one token is slot order, with their
// gate weights, then the shared expert).
template <int LPR>
__global__ __launch_bounds__(64 * kDecMaxSlots) void k_down_narrow_dec1(LayerDev L, Dims D,
                                                                        const float *__restrict__ h, UnionDev U,
                                                                        const float *__restrict__ w,
                                                                        float *__restrict__ residual) {
  using NS = NarrowShape<LPR>;
  __shared__ float vb[kDecMaxSlots][kTileRows];
  __shared__ int ok_s[kDecMaxSlots];
  __shared__ float wsl_s[kDecMaxSlots];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ti = blockIdx.x;
  const int nu = clamp_nu(U.n_unique, D);
  const int slots = nu + D.n_shared;
  float rin = 0.0f;
  if (wave == 0) {
    // slot lane's gate weight: its one pair's top-k position (pair = slot)
    float wv = 0.0f;
    if (lane < nu) {
      int js = U.pair_slot[lane];
      js = js < 0 ? 0 : (js >= D.k ? D.k - 1 : js);  // caller-supplied lists stay in bounds
      wv = w[js];
    }
    if (lane < kDecMaxSlots) wsl_s[lane] = wv;
    rin = residual[(size_t)ti * kTileRows + (lane & 7)];
  }
  if (wave < slots) {
    int e, p0, p1;
    const bool ok = resolve_slot(D, U, nu, wave, e, p0, p1) && p1 > p0;
    if (__builtin_amdgcn_readfirstlane((int)ok)) {
      const ExpertLayout EL = expert_layout(D.d, D.f);
      const uint8_t *base = expert_base(L, e);
      const int xrow[1] = {wave < nu ? p0 : D.T * D.k};
      float acc[1][NS::RPG];
      narrow_tile<LPR, 1>(base + EL.dn_nib, base + EL.dn_sc, ti, D.f, h, (size_t)D.f, xrow, 1, acc);
      narrow_reduce<LPR>(acc[0], vb[wave]);
    }
    if (lane == 0) ok_s[wave] = ok;
  }
  __syncthreads();
  if (wave == 0 && lane < kTileRows) {
    float out = rin;
    for (int sl = 0; sl < slots; ++sl) {
      if (!ok_s[sl]) continue;
      const float v = vb[sl][lane];
      out = sl < nu ? __builtin_fmaf(wsl_s[sl], v, out) : out + v;
    }
    residual[(size_t)ti * kTileRows + lane] = out;
  }
}

// ------------------------------------------------------------------ combine
// A7: r[t] += sum over the token's experts in ascending id of w * y, then the
// shared expert's y (weight 1).  Fixed order, no atomics: a token's result
// is the same whether it runs alone or batched, fused or not.

__global__ __launch_bounds__(256) void k_combine(Dims D, const float *__restrict__ w, UnionDev U,
                                                 const float *__restrict__ y, float *__restrict__ residual) {
  // Block (column slice, token): 256 threads x 4 columns.  A token's pairs sit
  // in ascending expert order in the union lists, so visiting its slots by
  // increasing pair index visits experts ascending; the order is ranked into
  // LDS by every block of the token.
  __shared__ int order[16];
  __shared__ float wt[16];
  __shared__ int nsel;
  const int t = blockIdx.y;
  if (t >= D.T) return;
  const int nu = clamp_nu(U.n_unique, D);
  const int tk = D.T * D.k;
  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    int p = 0x7FFFFFFF;
    if (nu > 0 && j < D.k) {
      p = U.pair_of[(size_t)t * D.k + j];
      if (p < 0 || p >= tk) p = 0x7FFFFFFF;
    }
    int rank = 0, valid = 0;
    for (int i = 0; i < D.k; ++i) {
      const int q = __shfl(p, i, 64);
      rank += (q < p) || (q == p && i < j);
      valid += q < tk;
    }
    if (j < D.k && p < tk) {
      order[rank] = p;
      wt[rank] = w[(size_t)t * D.k + j];
    }
    if (j == 0) nsel = valid;
  }
  __syncthreads();
  const int n = nsel;
  const int d4 = D.d / 4, c4 = blockIdx.x * 256 + threadIdx.x;
  if (c4 >= d4) return;
  float4 *rp = (float4 *)residual + (size_t)t * d4 + c4;
  const float4 *y4 = (const float4 *)y;
  float4 acc = *rp;
  if (n > 0) {
    // every load first (a slot past n reads the last valid row again), then
    // the fmas in slot order
    float4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i < D.k) v[i] = y4[(size_t)order[i < n ? i : n - 1] * d4 + c4];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i < n) {
        const float a = wt[i];
        acc.x = __builtin_fmaf(a, v[i].x, acc.x);
        acc.y = __builtin_fmaf(a, v[i].y, acc.y);
        acc.z = __builtin_fmaf(a, v[i].z, acc.z);
        acc.w = __builtin_fmaf(a, v[i].w, acc.w);
      }
  }
  if (D.n_shared) {
    const float4 sh = y4[((size_t)tk + t) * d4 + c4];
    acc.x = acc.x + sh.x;
    acc.y = acc.y + sh.y;
    acc.z = acc.z + sh.z;
    acc.w = acc.w + sh.w;
  }
  *rp = acc;
}

// ------------------------------------------------------------------ rmsnorm
// x = r / sqrt(mean(r^2) + eps), unit weight; one block of 512 threads per
// token, 16-byte loads, fixed reduction order (per thread in column order,
// then the wave tree, then the 8 waves in order).

__global__ __launch_bounds__(512) void k_rmsnorm(const float *__restrict__ r, int d, float eps,
                                                 float *__restrict__ x) {
  __shared__ float part[8];
  const int t = blockIdx.x;
  const float4 *rr = (const float4 *)(r + (size_t)t * d);
  float4 *xx = (float4 *)(x + (size_t)t * d);
  const int n4 = d / 4;
  float4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = threadIdx.x + 512 * i;
    v[i] = c < n4 ? rr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc = __builtin_fmaf(v[i].x, v[i].x, acc);
    acc = __builtin_fmaf(v[i].y, v[i].y, acc);
    acc = __builtin_fmaf(v[i].z, v[i].z, acc);
    acc = __builtin_fmaf(v[i].w, v[i].w, acc);
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  const float ss = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = threadIdx.x + 512 * i;
    if (c < n4) xx[c] = make_float4(v[i].x * inv, v[i].y * inv, v[i].z * inv, v[i].w * inv);
  }
}

// ---------------------------------------------------------------- launchers

static int slots_max(const Dims &D) {
  const long long tk = (long long)D.T * D.k;
  return (int)(tk < D.E ? tk : D.E) + D.n_shared;
}

static int topk_per(int E) {
  const int per = (E + 63) / 64;
  return per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : 16;
}

hipError_t launch_router_split(const LayerDev &L, const Dims &D, const float *x, float *logits, uint32_t *xq,
                               float *xs, hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  k_router_split<false><<<D.E, 256, 0, s>>>(L, D, x, logits, xq, xs, 0.0f, nullptr);
  return hipGetLastError();
}

hipError_t launch_router_norm(const LayerDev &L, const Dims &D, const float *r, float eps, float *xout, float *logits,
                              uint32_t *xq, float *xs, hipStream_t s) {
  if (D.T != 1 || D.d > 8 * 512 * 4) return hipErrorInvalidValue;
  k_router_split<true><<<D.E, 256, 0, s>>>(L, D, r, logits, xq, xs, eps, xout);
  return hipGetLastError();
}

hipError_t launch_topk_union1(const float *logits, const Dims &D, int32_t *idx, float *w, const UnionDev *U,
                              float top_p, hipStream_t s) {
  const UnionDev u = U ? *U : UnionDev{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  const int wu = U ? 1 : 0;
  switch (topk_per(D.E)) {
    case 1: k_topk_union1<1><<<1, 64, 0, s>>>(logits, D, idx, w, u, wu, top_p); break;
    case 2: k_topk_union1<2><<<1, 64, 0, s>>>(logits, D, idx, w, u, wu, top_p); break;
    case 4: k_topk_union1<4><<<1, 64, 0, s>>>(logits, D, idx, w, u, wu, top_p); break;
    case 8: k_topk_union1<8><<<1, 64, 0, s>>>(logits, D, idx, w, u, wu, top_p); break;
    default: k_topk_union1<16><<<1, 64, 0, s>>>(logits, D, idx, w, u, wu, top_p); break;
  }
  return hipGetLastError();
}

bool route_one_small_supported(const Dims &D) {
  const int nf = (D.d / 4 + 255) / 256;
  return D.T == 1 && D.E <= kRouteOneMaxE && nf <= 2;
}

hipError_t launch_route_one_small(const LayerDev &L, const Dims &D, const float *x, float *logits, int32_t *idx,
                                  float *w, const UnionDev *U, float top_p, hipStream_t s) {
  if (!route_one_small_supported(D)) return hipErrorInvalidValue;
  const UnionDev u = U ? *U : UnionDev{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  const int wu = U ? 1 : 0;
  // E <= 32: one top-k key per lane (topk_per(E) = 1)
  if ((D.d / 4 + 255) / 256 == 1)
    k_route_one_small<1, 1><<<1, 1024, 0, s>>>(L, D, x, logits, idx, w, u, wu, top_p);
  else
    k_route_one_small<2, 1><<<1, 1024, 0, s>>>(L, D, x, logits, idx, w, u, wu, top_p);
  return hipGetLastError();
}

bool shared_early_supported(const Dims &D) {
  const int NS = (D.d / kChunk + 63) / 64;
  return D.T == 1 && D.n_shared == 1 && NS <= 4 && D.f % 16 == 0;
}

template <int PER>
static void topk_shared1_launch(int NS, int grid, hipStream_t s, const float *logits, const Dims &D, int32_t *idx,
                                float *w, const UnionDev &u, int wu, float top_p, const LayerDev &L,
                                const uint32_t *xq, const float *xs, uint32_t *hq, float *hs) {
  switch (NS) {
    case 1: k_topk_shared1<PER, 1><<<grid, 256, 0, s>>>(logits, D, idx, w, u, wu, top_p, L, xq, xs, hq, hs); break;
    case 2: k_topk_shared1<PER, 2><<<grid, 512, 0, s>>>(logits, D, idx, w, u, wu, top_p, L, xq, xs, hq, hs); break;
    case 3: k_topk_shared1<PER, 3><<<grid, 768, 0, s>>>(logits, D, idx, w, u, wu, top_p, L, xq, xs, hq, hs); break;
    default: k_topk_shared1<PER, 4><<<grid, 1024, 0, s>>>(logits, D, idx, w, u, wu, top_p, L, xq, xs, hq, hs); break;
  }
}

hipError_t launch_topk_shared1(const float *logits, const Dims &D, int32_t *idx, float *w, const UnionDev *U,
                               float top_p, const LayerDev &L, const uint32_t *xq, const float *xs, uint32_t *hq,
                               float *hs, hipStream_t s) {
  if (!shared_early_supported(D)) return hipErrorInvalidValue;
  const UnionDev u = U ? *U : UnionDev{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  const int wu = U ? 1 : 0;
  const int NS = (D.d / kChunk + 63) / 64, grid = 1 + D.f / 16;
  switch (topk_per(D.E)) {
    case 1: topk_shared1_launch<1>(NS, grid, s, logits, D, idx, w, u, wu, top_p, L, xq, xs, hq, hs); break;
    case 2: topk_shared1_launch<2>(NS, grid, s, logits, D, idx, w, u, wu, top_p, L, xq, xs, hq, hs); break;
    case 4: topk_shared1_launch<4>(NS, grid, s, logits, D, idx, w, u, wu, top_p, L, xq, xs, hq, hs); break;
    case 8: topk_shared1_launch<8>(NS, grid, s, logits, D, idx, w, u, wu, top_p, L, xq, xs, hq, hs); break;
    default: topk_shared1_launch<16>(NS, grid, s, logits, D, idx, w, u, wu, top_p, L, xq, xs, hq, hs); break;
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float *logits, const Dims &D, int32_t *idx, float *w, float top_p, hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  dim3 g((D.T + 3) / 4), b(256);
  switch (topk_per(D.E)) {
    case 1: k_topk<1><<<g, b, 0, s>>>(logits, D, idx, w, top_p); break;
    case 2: k_topk<2><<<g, b, 0, s>>>(logits, D, idx, w, top_p); break;
    case 4: k_topk<4><<<g, b, 0, s>>>(logits, D, idx, w, top_p); break;
    case 8: k_topk<8><<<g, b, 0, s>>>(logits, D, idx, w, top_p); break;
    default: k_topk<16><<<g, b, 0, s>>>(logits, D, idx, w, top_p); break;
  }
  return hipGetLastError();
}

// Union lists of a call with at most 64 (token, slot) pairs, one wave: lane p
// holds pair p and ranks it by (expert, token) among all pairs with a plain
// count; the lists (and the handling of an invalid routing) are those of
// union_wave.  idx may point to LDS (the top-k's copy of the routing).
__device__ void union_small(const int32_t *__restrict__ idx, const Dims &D, const UnionDev &U,
                            int32_t *__restrict__ err) {
  const int P = D.T * D.k, lane = threadIdx.x & 63;
  const bool act = lane < P;
  const int e = act ? idx[lane] : 0;
  const int t = act ? lane / D.k : 0, j = act ? lane - t * D.k : 0;
  const bool live = act && e != kDropped;  // a slot dropped by expert top-p has no pair
  bool ok = !live || (e >= 0 && e < D.E);
  // distinct within the token: compare with the ids of slots 0..j-1 of the
  // same token, taken from the lanes that hold them
  for (int q = 0; q + 1 < D.k; ++q) {
    const int eq = __shfl(e, t * D.k + q, 64);
    if (live && q < j && eq == e) ok = false;
  }
  if (__ballot(!ok)) {
    if (lane == 0) {
      *U.n_unique = 0;
      U.offsets[0] = 0;
      atomicOr(err, 1);
    }
    return;
  }
  const int key = live ? e * D.T + t : 0x7FFFFFFF;  // (expert, token), unique per pair
  int rank = 0;
  bool first = live;
  for (int q = 0; q < P; ++q) {
    const int kq = __shfl(key, q, 64), eq = __shfl(e, q, 64);
    rank += kq < key;
    first = first && !(eq == e && kq < key);
  }
  const unsigned long long fm = __ballot(first);
  int below = 0;  // distinct experts smaller than e
  for (int q = 0; q < P; ++q) below += ((fm >> q) & 1ull) && __shfl(e, q, 64) < e;
  const int kept = __popcll(__ballot(live));
  if (live) {
    U.pair_token[rank] = t;
    U.pair_slot[rank] = j;
    U.pair_of[lane] = rank;
    if (first) {
      U.ids[below] = e;
      U.offsets[below] = rank;
    }
  } else if (act) {
    U.pair_of[lane] = -1;
  }
  if (lane == 0) {
    const int n = __popcll(fm);
    *U.n_unique = n;
    U.offsets[n] = kept;
  }
}

// Top-k of up to 16 tokens (one wave each) and their union lists (wave 0,
// after the block barrier) in one launch; the same functions as k_topk and
// k_union, so the same results.
template <int PER>
__global__ __launch_bounds__(1024) void k_topk_union(const float *__restrict__ logits, Dims D,
                                                     int32_t *__restrict__ idx, float *__restrict__ wout, UnionDev U,
                                                     int32_t *__restrict__ err, float top_p) {
  extern __shared__ unsigned long long masks[];
  __shared__ int32_t sids[kRouteSplitMaxT * 16];  // the call's routing (T <= 16, k <= 16) for the union
  const int t = threadIdx.x >> 6;
  if (t < D.T) topk_token<PER>(logits + (size_t)t * D.E, D, t, idx, wout, sids, top_p);
  __syncthreads();
  if (threadIdx.x < 64) {
    if (D.T * D.k <= 64)
      union_small(sids, D, U, err);
    else
      union_wave(sids, D, U, err, masks);
  }
}

// As k_topk_union (block 0), and beside it the shared expert's gate/up for
// every token (blocks 1.., one (quad, token) item each, the one-token block
// code): the shared expert does not depend on the routing, so its weights
// stream while the selection runs.  Items are quad-major with XCD-contiguous
// ranges, as in k_gateup_pairs, so the tokens of one quad share an L2.
template <int PER, int NS>
__global__ __launch_bounds__(1024) void k_topk_union_shared(const float *__restrict__ logits, Dims D,
                                                            int32_t *__restrict__ idx, float *__restrict__ wout,
                                                            UnionDev U, int32_t *__restrict__ err, float top_p,
                                                            LayerDev L, const uint32_t *__restrict__ xq,
                                                            const float *__restrict__ xs, uint32_t *__restrict__ hq,
                                                            float *__restrict__ hs) {
  extern __shared__ unsigned long long masks[];
  __shared__ int32_t sids[kRouteSplitMaxT * 16];
  if (blockIdx.x > 0) {
    if ((int)threadIdx.x >= 256 * NS) return;  // waves past the block code's
    const int b = (int)blockIdx.x - 1, per = ((int)gridDim.x - 1) / 8;
    const int item = (b % 8) * per + b / 8;
    if (item >= D.T * (D.f / 16)) return;  // block-uniform
    const int qd = item / D.T, t = item - qd * D.T;
    gateup_one_quad<NS>(L, D, D.E, D.T * D.k + t, qd, t, xq, xs, hq, hs);
    return;
  }
  const int t = threadIdx.x >> 6;
  if (t < D.T) topk_token<PER>(logits + (size_t)t * D.E, D, t, idx, wout, sids, top_p);
  __syncthreads();
  if (threadIdx.x < 64) {
    if (D.T * D.k <= 64)
      union_small(sids, D, U, err);
    else
      union_wave(sids, D, U, err, masks);
  }
}

bool shared_early_multi_supported(const Dims &D) {
  const int NS = (D.d / kChunk + 63) / 64;
  return D.T >= 2 && D.T <= kSharedEarlyMaxT && D.n_shared == 1 && NS <= 4 && D.f % 16 == 0;
}

template <int PER>
static void topk_union_shared_launch(int NS, int grid, int block, size_t lds, hipStream_t s, const float *logits,
                                     const Dims &D, int32_t *idx, float *w, const UnionDev &U, int32_t *err,
                                     float top_p, const LayerDev &L, const uint32_t *xq, const float *xs,
                                     uint32_t *hq, float *hs) {
  switch (NS) {
    case 1: k_topk_union_shared<PER, 1><<<grid, block, lds, s>>>(logits, D, idx, w, U, err, top_p, L, xq, xs, hq, hs); break;
    case 2: k_topk_union_shared<PER, 2><<<grid, block, lds, s>>>(logits, D, idx, w, U, err, top_p, L, xq, xs, hq, hs); break;
    case 3: k_topk_union_shared<PER, 3><<<grid, block, lds, s>>>(logits, D, idx, w, U, err, top_p, L, xq, xs, hq, hs); break;
    default: k_topk_union_shared<PER, 4><<<grid, block, lds, s>>>(logits, D, idx, w, U, err, top_p, L, xq, xs, hq, hs); break;
  }
}

hipError_t launch_topk_union_shared(const float *logits, const Dims &D, int32_t *idx, float *w, const UnionDev &U,
                                    int32_t *err, float top_p, const LayerDev &L, const uint32_t *xq,
                                    const float *xs, uint32_t *hq, float *hs, hipStream_t s) {
  if (!shared_early_multi_supported(D)) return hipErrorInvalidValue;
  const int NS = (D.d / kChunk + 63) / 64;
  const int block = 64 * D.T > 256 * NS ? 64 * D.T : 256 * NS;
  const int grid = 1 + 8 * ((D.T * (D.f / 16) + 7) / 8);
  const size_t lds = union_lds_bytes(D.E);
  switch (topk_per(D.E)) {
    case 1: topk_union_shared_launch<1>(NS, grid, block, lds, s, logits, D, idx, w, U, err, top_p, L, xq, xs, hq, hs); break;
    case 2: topk_union_shared_launch<2>(NS, grid, block, lds, s, logits, D, idx, w, U, err, top_p, L, xq, xs, hq, hs); break;
    case 4: topk_union_shared_launch<4>(NS, grid, block, lds, s, logits, D, idx, w, U, err, top_p, L, xq, xs, hq, hs); break;
    case 8: topk_union_shared_launch<8>(NS, grid, block, lds, s, logits, D, idx, w, U, err, top_p, L, xq, xs, hq, hs); break;
    default: topk_union_shared_launch<16>(NS, grid, block, lds, s, logits, D, idx, w, U, err, top_p, L, xq, xs, hq, hs); break;
  }
  return hipGetLastError();
}

hipError_t launch_topk_union(const float *logits, const Dims &D, int32_t *idx, float *w, const UnionDev &U,
                             int32_t *err, float top_p, hipStream_t s) {
  if (D.T < 1 || D.T > kRouteSplitMaxT) return hipErrorInvalidValue;
  const int b = 64 * D.T;
  const size_t lds = union_lds_bytes(D.E);
  switch (topk_per(D.E)) {
    case 1: k_topk_union<1><<<1, b, lds, s>>>(logits, D, idx, w, U, err, top_p); break;
    case 2: k_topk_union<2><<<1, b, lds, s>>>(logits, D, idx, w, U, err, top_p); break;
    case 4: k_topk_union<4><<<1, b, lds, s>>>(logits, D, idx, w, U, err, top_p); break;
    case 8: k_topk_union<8><<<1, b, lds, s>>>(logits, D, idx, w, U, err, top_p); break;
    default: k_topk_union<16><<<1, b, lds, s>>>(logits, D, idx, w, U, err, top_p); break;
  }
  return hipGetLastError();
}

hipError_t launch_union(const int32_t *idx, const Dims &D, const UnionDev &U, int32_t *err, hipStream_t s) {
  if (D.T > 256) {
    // one wave per segment; LDS stays under 64 KB
    int W = 16;
    while (W > 1 && union_multi_lds_bytes(D.E, W) > 64 * 1024) W >>= 1;
    k_union_multi<<<1, 64 * W, union_multi_lds_bytes(D.E, W), s>>>(idx, D, U, err);
  } else {
    k_union<<<1, 64, union_lds_bytes(D.E), s>>>(idx, D, U, err);
  }
  return hipGetLastError();
}

static bool wide(int K) { return K / kChunk >= 64; }

// Lanes per row of the narrow kernels: every lane takes one 32-column chunk,
// so a row needs at least as many lanes as it has chunks.
static int narrow_lpr(int K) {
  const int C = K / kChunk;
  return C > 32 ? 64 : C > 16 ? 32 : C > 8 ? 16 : C > 4 ? 8 : C > 2 ? 4 : 2;
}

static int grid_cap(long long blocks, int cap) { return (int)(blocks < 1 ? 1 : blocks > cap ? cap : blocks); }

template <int LPR>
static void narrow_gateup(bool mt1, int grid, hipStream_t s, const LayerDev &L, const Dims &D, const float *x,
                          const UnionDev &U, float *h, float *g, float *u) {
  if (mt1)
    k_gateup_narrow<LPR, 1><<<grid, 256, 0, s>>>(L, D, x, U, h, g, u);
  else
    k_gateup_narrow<LPR, 8><<<grid, 256, 0, s>>>(L, D, x, U, h, g, u);
}

template <int LPR>
static void narrow_down(bool mt1, int grid, hipStream_t s, const LayerDev &L, const Dims &D, const float *h,
                        const UnionDev &U, float *y) {
  if (mt1)
    k_down_narrow<LPR, 1><<<grid, 256, 0, s>>>(L, D, h, U, y);
  else
    k_down_narrow<LPR, 8><<<grid, 256, 0, s>>>(L, D, h, U, y);
}

static hipError_t gateup_impl(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h, float *g,
                              float *u, hipStream_t s) {
  const bool mt1 = D.T == 1;
  const long long items = (long long)slots_max(D) * (D.f / 4);
  if (wide(D.d)) {
    const int nw = (D.d / kChunk + 63) / 64;
    dim3 grid(grid_cap(items, 16384)), block(64 * nw);
    if (mt1)
      k_gateup_wide<1><<<grid, block, 0, s>>>(L, D, x, U, h, g, u);
    else
      k_gateup_wide<8><<<grid, block, 0, s>>>(L, D, x, U, h, g, u);
  } else {
    const int grid = grid_cap((items + 3) / 4, 8192);
    switch (narrow_lpr(D.d)) {
      case 64: narrow_gateup<64>(mt1, grid, s, L, D, x, U, h, g, u); break;
      case 32: narrow_gateup<32>(mt1, grid, s, L, D, x, U, h, g, u); break;
      case 16: narrow_gateup<16>(mt1, grid, s, L, D, x, U, h, g, u); break;
      case 8: narrow_gateup<8>(mt1, grid, s, L, D, x, U, h, g, u); break;
      case 4: narrow_gateup<4>(mt1, grid, s, L, D, x, U, h, g, u); break;
      default: narrow_gateup<2>(mt1, grid, s, L, D, x, U, h, g, u); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_gateup(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h,
                         hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  return gateup_impl(L, D, x, U, h, nullptr, nullptr, s);
}

hipError_t launch_debug_gateup(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h,
                               float *g, float *u, hipStream_t s) {
  return gateup_impl(L, D, x, U, h, g, u, s);
}

// Rows of y the fused down kernel keeps in LDS (pairs plus shared rows).
static size_t fused_rows(const Dims &D) { return (size_t)D.T * D.k + (size_t)D.T * D.n_shared; }

bool down_fusable(const Dims &D) { return wide(D.f) && fused_rows(D) * kTileRows * 4 <= kFusedLdsMax; }

bool narrow_dec_supported(const Dims &D) { return D.T == 1 && !wide(D.f) && slots_max(D) <= kDecMaxSlots; }

hipError_t launch_down(const LayerDev &L, const Dims &D, const float *h, const UnionDev &U, float *y,
                       const float *w, float *residual, bool fused, hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  const bool mt1 = D.T == 1;
  if (wide(D.f)) {
    const int tiles = D.d / kTileRows;
    const int nwmax = mt1 ? 9 : 8;  // decode: k = 8 routed + shared slots side by side
    int nw = slots_max(D);
    nw = nw < 1 ? 1 : nw > nwmax ? nwmax : nw;
    dim3 grid(tiles), block(64 * nw);
    const size_t lds = fused ? fused_rows(D) * kTileRows * 4 : 0;
    if (fused) {
      if (mt1)
        k_down_wide<1, true, 9><<<grid, block, lds, s>>>(L, D, h, U, y, w, residual);
      else
        k_down_wide<8, true, 8><<<grid, block, lds, s>>>(L, D, h, U, y, w, residual);
    } else {
      if (mt1)
        k_down_wide<1, false, 9><<<grid, block, 0, s>>>(L, D, h, U, y, w, residual);
      else
        k_down_wide<8, false, 8><<<grid, block, 0, s>>>(L, D, h, U, y, w, residual);
    }
  } else if (fused) {  // one token (narrow_dec_supported)
    const dim3 grid(D.d / kTileRows), block(64 * slots_max(D));
    switch (narrow_lpr(D.f)) {
      case 64: k_down_narrow_dec1<64><<<grid, block, 0, s>>>(L, D, h, U, w, residual); break;
      case 32: k_down_narrow_dec1<32><<<grid, block, 0, s>>>(L, D, h, U, w, residual); break;
      case 16: k_down_narrow_dec1<16><<<grid, block, 0, s>>>(L, D, h, U, w, residual); break;
      case 8: k_down_narrow_dec1<8><<<grid, block, 0, s>>>(L, D, h, U, w, residual); break;
      case 4: k_down_narrow_dec1<4><<<grid, block, 0, s>>>(L, D, h, U, w, residual); break;
      default: k_down_narrow_dec1<2><<<grid, block, 0, s>>>(L, D, h, U, w, residual); break;
    }
  } else {
    const long long items = (long long)slots_max(D) * (D.d / kTileRows);
    const int grid = grid_cap((items + 3) / 4, 8192);
    switch (narrow_lpr(D.f)) {
      case 64: narrow_down<64>(mt1, grid, s, L, D, h, U, y); break;
      case 32: narrow_down<32>(mt1, grid, s, L, D, h, U, y); break;
      case 16: narrow_down<16>(mt1, grid, s, L, D, h, U, y); break;
      case 8: narrow_down<8>(mt1, grid, s, L, D, h, U, y); break;
      case 4: narrow_down<4>(mt1, grid, s, L, D, h, U, y); break;
      default: narrow_down<2>(mt1, grid, s, L, D, h, U, y); break;
    }
  }
  return hipGetLastError();
}

bool fxp_supported(const Dims &D) { return wide(D.d) && wide(D.f); }

hipError_t launch_xquant(const float *x, int T, int K, uint32_t *xq, float *xs, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const long long groups = (long long)T * (K / 16);
  k_xquant<<<grid_cap((groups + 255) / 256, 4096), 256, 0, s>>>(x, T, K, xq, xs);
  return hipGetLastError();
}

static size_t tok_lds(int K) {
  const int NS = (K / kChunk + 63) / 64;
  return (size_t)4 * NS * kTokChunk * kTileRows * 4;
}

template <int SPW, bool ONE>
static void gateup_tok_launch(int wpt, int grid, size_t lds, hipStream_t s, const LayerDev &L, const Dims &D,
                              const UnionDev &U, const float *w, const uint32_t *xq, const float *xs, uint32_t *hq,
                              float *hs, float *wslot) {
  switch (wpt) {
    case 1: k_gateup_tok<SPW, ONE, 1><<<grid, 256, lds, s>>>(L, D, U, w, xq, xs, hq, hs, wslot); break;
    case 2: k_gateup_tok<SPW, ONE, 2><<<grid, 512, lds, s>>>(L, D, U, w, xq, xs, hq, hs, wslot); break;
    case 3: k_gateup_tok<SPW, ONE, 3><<<grid, 768, lds, s>>>(L, D, U, w, xq, xs, hq, hs, wslot); break;
    default: k_gateup_tok<SPW, ONE, 4><<<grid, 1024, lds, s>>>(L, D, U, w, xq, xs, hq, hs, wslot); break;
  }
}

template <int SPW, bool ONE>
static void down_tok_launch(int wpt, int grid, size_t lds, hipStream_t s, const LayerDev &L, const Dims &D,
                            const UnionDev &U, const uint32_t *hq, const float *hs, float *y) {
  switch (wpt) {
    case 1: k_down_tok<SPW, ONE, 1><<<grid, 256, lds, s>>>(L, D, U, hq, hs, y); break;
    case 2: k_down_tok<SPW, ONE, 2><<<grid, 512, lds, s>>>(L, D, U, hq, hs, y); break;
    case 3: k_down_tok<SPW, ONE, 3><<<grid, 768, lds, s>>>(L, D, U, hq, hs, y); break;
    default: k_down_tok<SPW, ONE, 4><<<grid, 1024, lds, s>>>(L, D, U, hq, hs, y); break;
  }
}

hipError_t launch_gateup_tok(const LayerDev &L, const Dims &D, const UnionDev &U, const int32_t *idx, const float *w,
                             const uint32_t *xq, const float *xs, uint32_t *hq, float *hs, float *wslot,
                             bool skip_shared, hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  const int NS = (D.d / kChunk + 63) / 64, wpt = NS < 4 ? NS : 4;
  const int slots = (D.T * D.k < D.E ? D.T * D.k : D.E) + D.n_shared;
  int grid = slots * (D.f / 16);
  const size_t lds = tok_lds(D.d);
  if (D.T == 1) {
    if (skip_shared && NS <= 4) grid -= D.n_shared * (D.f / 16);  // the shared expert's blocks would only exit
    if (NS <= 4) {
      switch (NS) {
        case 1: k_gateup_one<1><<<grid, 256, 0, s>>>(L, D, U, w, xq, xs, hq, hs, wslot, skip_shared ? 1 : 0); break;
        case 2: k_gateup_one<2><<<grid, 512, 0, s>>>(L, D, U, w, xq, xs, hq, hs, wslot, skip_shared ? 1 : 0); break;
        case 3: k_gateup_one<3><<<grid, 768, 0, s>>>(L, D, U, w, xq, xs, hq, hs, wslot, skip_shared ? 1 : 0); break;
        default: k_gateup_one<4><<<grid, 1024, 0, s>>>(L, D, U, w, xq, xs, hq, hs, wslot, skip_shared ? 1 : 0); break;
      }
    } else
      gateup_tok_launch<2, true>(wpt, grid, lds, s, L, D, U, w, xq, xs, hq, hs, wslot);
  } else if (NS <= 4 && D.T <= kPairsMaxT) {
    // with skip_shared the shared expert's rows are already there
    const int items = (D.T * D.k + (skip_shared ? 0 : D.T * D.n_shared)) * (D.f / 16);
    const int pgrid = 8 * ((items + 7) / 8);
    switch (NS) {
      case 1: k_gateup_pairs<1><<<pgrid, 256, 0, s>>>(L, D, U, idx, xq, xs, hq, hs, items); break;
      case 2: k_gateup_pairs<2><<<pgrid, 512, 0, s>>>(L, D, U, idx, xq, xs, hq, hs, items); break;
      case 3: k_gateup_pairs<3><<<pgrid, 768, 0, s>>>(L, D, U, idx, xq, xs, hq, hs, items); break;
      default: k_gateup_pairs<4><<<pgrid, 1024, 0, s>>>(L, D, U, idx, xq, xs, hq, hs, items); break;
    }
  } else {
    if (NS <= 4)
      gateup_tok_launch<1, false>(wpt, grid, lds, s, L, D, U, w, xq, xs, hq, hs, wslot);
    else
      gateup_tok_launch<2, false>(wpt, grid, lds, s, L, D, U, w, xq, xs, hq, hs, wslot);
  }
  return hipGetLastError();
}

hipError_t launch_down_tok(const LayerDev &L, const Dims &D, const UnionDev &U, const uint32_t *hq, const float *hs,
                           float *y, hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  const int NS = (D.f / kChunk + 63) / 64, wpt = NS < 4 ? NS : 4;
  const int slots = (D.T * D.k < D.E ? D.T * D.k : D.E) + D.n_shared;
  const int grid = slots * (D.d / 32);
  const size_t lds = tok_lds(D.f);
  if (D.T == 1) {
    if (NS <= 4)
      down_tok_launch<1, true>(wpt, grid, lds, s, L, D, U, hq, hs, y);
    else
      down_tok_launch<2, true>(wpt, grid, lds, s, L, D, U, hq, hs, y);
  } else {
    if (NS <= 4)
      down_tok_launch<1, false>(wpt, grid, lds, s, L, D, U, hq, hs, y);
    else
      down_tok_launch<2, false>(wpt, grid, lds, s, L, D, U, hq, hs, y);
  }
  return hipGetLastError();
}

bool f32_dec_supported(const Dims &D) {
  const int NS = (D.d / kChunk + 63) / 64;
  return D.T == 1 && wide(D.d) && NS <= 4 && D.f % (16 * kF32DecTPW) == 0 && down_fusable(D) &&
         D.k + D.n_shared <= kDecMaxSlots;
}

hipError_t launch_gateup_f32_dec(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h,
                                 float *hsum, hipStream_t s) {
  if (!f32_dec_supported(D)) return hipErrorInvalidValue;
  const int NS = (D.d / kChunk + 63) / 64;
  const int grid = slots_max(D) * (D.f / (16 * kF32DecTPW));
  switch (NS) {
    case 1: k_gateup_f32_dec<1, kF32DecTPW, false><<<grid, 256, 0, s>>>(L, D, x, U, h, hsum, nullptr, 0); break;
    case 2: k_gateup_f32_dec<2, kF32DecTPW, false><<<grid, 256, 0, s>>>(L, D, x, U, h, hsum, nullptr, 0); break;
    case 3: k_gateup_f32_dec<3, kF32DecTPW, false><<<grid, 256, 0, s>>>(L, D, x, U, h, hsum, nullptr, 0); break;
    default: k_gateup_f32_dec<4, kF32DecTPW, false><<<grid, 256, 0, s>>>(L, D, x, U, h, hsum, nullptr, 0); break;
  }
  return hipGetLastError();
}

bool f32_dec_tok_supported(const Dims &D) {
  const int NS = (D.d / kChunk + 63) / 64;
  return D.T >= 2 && D.T <= kF32TokMaxT && wide(D.d) && NS <= 4 && D.f % (16 * kF32DecTPW) == 0 &&
         down_fusable(D) && D.k + D.n_shared <= kDecMaxSlots;
}

hipError_t launch_f32_dec_tok(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U,
                              const int32_t *idx, const float *w, float *h, float *hsum, float *residual,
                              hipStream_t s) {
  if (!f32_dec_tok_supported(D)) return hipErrorInvalidValue;
  const int NS = (D.d / kChunk + 63) / 64;
  const int gitems = (D.T * D.k + D.T * D.n_shared) * (D.f / (16 * kF32DecTPW));
  const int ggrid = 8 * ((gitems + 7) / 8);
  switch (NS) {
    case 1: k_gateup_f32_dec<1, kF32DecTPW, true><<<ggrid, 256, 0, s>>>(L, D, x, U, h, hsum, idx, gitems); break;
    case 2: k_gateup_f32_dec<2, kF32DecTPW, true><<<ggrid, 256, 0, s>>>(L, D, x, U, h, hsum, idx, gitems); break;
    case 3: k_gateup_f32_dec<3, kF32DecTPW, true><<<ggrid, 256, 0, s>>>(L, D, x, U, h, hsum, idx, gitems); break;
    default: k_gateup_f32_dec<4, kF32DecTPW, true><<<ggrid, 256, 0, s>>>(L, D, x, U, h, hsum, idx, gitems); break;
  }
  const int ditems = D.T * (D.d / kTileRows);
  k_down_f32_tok<<<8 * ((ditems + 7) / 8), 64 * (D.k + D.n_shared), 0, s>>>(L, D, h, hsum, U, idx, w, residual,
                                                                            ditems);
  return hipGetLastError();
}

hipError_t launch_down_f32_dec(const LayerDev &L, const Dims &D, const float *h, const float *hsum, const UnionDev &U,
                               const float *w, float *residual, hipStream_t s) {
  if (!f32_dec_supported(D)) return hipErrorInvalidValue;
  k_down_f32_dec<<<D.d / kTileRows, 64 * (D.k + D.n_shared), 0, s>>>(L, D, h, hsum, U, w, residual);
  return hipGetLastError();
}

bool down_dec_supported(const Dims &D) {
  return D.T == 1 && (D.f / kChunk + 63) / 64 == 1 && D.k + D.n_shared <= kDecMaxSlots;
}

bool down_dec_tok_supported(const Dims &D) {
  return D.T >= 2 && D.T <= kDownTokMaxT && (D.f / kChunk + 63) / 64 == 1 && D.k + D.n_shared <= kDecMaxSlots;
}

hipError_t launch_down_dec_tok(const LayerDev &L, const Dims &D, const uint32_t *hq, const float *hs,
                               const UnionDev &U, const int32_t *idx, const float *w, float *residual,
                               hipStream_t s) {
  if (!down_dec_tok_supported(D)) return hipErrorInvalidValue;
  const int items = D.T * (D.d / kTileRows);
  k_down_dec_tok<<<8 * ((items + 7) / 8), 64 * (D.k + D.n_shared), 0, s>>>(L, D, hq, hs, U, idx, w, residual,
                                                                            items);
  return hipGetLastError();
}

hipError_t launch_down_dec(const LayerDev &L, const Dims &D, const uint32_t *hq, const float *hs, const UnionDev &U,
                           const float *wslot, float *residual, hipStream_t s) {
  if (!down_dec_supported(D)) return hipErrorInvalidValue;
  k_down_dec1<<<D.d / kTileRows, 64 * (D.k + D.n_shared), 0, s>>>(L, D, hq, hs, U, wslot, residual);
  return hipGetLastError();
}

hipError_t launch_combine(const Dims &D, const float *w, const UnionDev &U, const float *y, float *residual,
                          hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  k_combine<<<dim3((D.d / 4 + 255) / 256, D.T), 256, 0, s>>>(D, w, U, y, residual);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float *r, int T, int d, float eps, float *x, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  k_rmsnorm<<<T, 512, 0, s>>>(r, d, eps, x);
  return hipGetLastError();
}

bool i8_dec_supported(const Dims &D) {
  const int gi = (D.d / 16 + 63) / 64, di = (D.f / 16 + 63) / 64;
  return D.T == 1 && D.d % kI8Rows == 0 && gi <= 8 && di <= 2 && D.k + D.n_shared <= kDecMaxSlots;
}

hipError_t launch_forward_i8_dec(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h,
                                 const float *w, float *residual, hipStream_t s) {
  if (!i8_dec_supported(D)) return hipErrorInvalidValue;
  const dim3 gg((D.f + 3) / 4, slots_max(D));
  switch ((D.d / 16 + 63) / 64) {
    case 1: k_gateup_i8_dec<1, false><<<gg, 256, 0, s>>>(L, D, x, U, h, nullptr, 0); break;
    case 2: k_gateup_i8_dec<2, false><<<gg, 256, 0, s>>>(L, D, x, U, h, nullptr, 0); break;
    case 3: k_gateup_i8_dec<3, false><<<gg, 256, 0, s>>>(L, D, x, U, h, nullptr, 0); break;
    case 4: k_gateup_i8_dec<4, false><<<gg, 256, 0, s>>>(L, D, x, U, h, nullptr, 0); break;
    case 5: k_gateup_i8_dec<5, false><<<gg, 256, 0, s>>>(L, D, x, U, h, nullptr, 0); break;
    case 6: k_gateup_i8_dec<6, false><<<gg, 256, 0, s>>>(L, D, x, U, h, nullptr, 0); break;
    case 7: k_gateup_i8_dec<7, false><<<gg, 256, 0, s>>>(L, D, x, U, h, nullptr, 0); break;
    default: k_gateup_i8_dec<8, false><<<gg, 256, 0, s>>>(L, D, x, U, h, nullptr, 0); break;
  }
  const int threads = 64 * (D.k + D.n_shared);
  if ((D.f / 16 + 63) / 64 == 1)
    k_down_i8_dec<1><<<D.d / kI8Rows, threads, 0, s>>>(L, D, h, U, w, residual);
  else
    k_down_i8_dec<2><<<D.d / kI8Rows, threads, 0, s>>>(L, D, h, U, w, residual);
  return hipGetLastError();
}

bool i8_tok_supported(const Dims &D) {
  const int gi = (D.d / 16 + 63) / 64, di = (D.f / 16 + 63) / 64;
  return D.T >= 2 && D.T <= kPairsMaxT && D.d % kI8Rows == 0 && gi <= 8 && di <= 2 &&
         D.k + D.n_shared <= kDecMaxSlots;
}

hipError_t launch_forward_i8_tok(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U,
                                 const int32_t *idx, float *h, const float *w, float *residual, hipStream_t s) {
  if (!i8_tok_supported(D)) return hipErrorInvalidValue;
  const int gitems = (D.T * D.k + D.T * D.n_shared) * ((D.f + 3) / 4);
  const int gg = 8 * ((gitems + 7) / 8);
  switch ((D.d / 16 + 63) / 64) {
    case 1: k_gateup_i8_dec<1, true><<<gg, 256, 0, s>>>(L, D, x, U, h, idx, gitems); break;
    case 2: k_gateup_i8_dec<2, true><<<gg, 256, 0, s>>>(L, D, x, U, h, idx, gitems); break;
    case 3: k_gateup_i8_dec<3, true><<<gg, 256, 0, s>>>(L, D, x, U, h, idx, gitems); break;
    case 4: k_gateup_i8_dec<4, true><<<gg, 256, 0, s>>>(L, D, x, U, h, idx, gitems); break;
    case 5: k_gateup_i8_dec<5, true><<<gg, 256, 0, s>>>(L, D, x, U, h, idx, gitems); break;
    case 6: k_gateup_i8_dec<6, true><<<gg, 256, 0, s>>>(L, D, x, U, h, idx, gitems); break;
    case 7: k_gateup_i8_dec<7, true><<<gg, 256, 0, s>>>(L, D, x, U, h, idx, gitems); break;
    default: k_gateup_i8_dec<8, true><<<gg, 256, 0, s>>>(L, D, x, U, h, idx, gitems); break;
  }
  const int ditems = D.T * (D.d / kI8Rows);
  const int dg = 8 * ((ditems + 7) / 8), threads = 64 * (D.k + D.n_shared);
  if ((D.f / 16 + 63) / 64 == 1)
    k_down_i8_tok<1><<<dg, threads, 0, s>>>(L, D, h, U, idx, w, residual, ditems);
  else
    k_down_i8_tok<2><<<dg, threads, 0, s>>>(L, D, h, U, idx, w, residual, ditems);
  return hipGetLastError();
}

hipError_t launch_forward_i8(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h, float *y,
                             hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  const int slots = slots_max(D);
  if (D.T == 1) {
    k_gateup_i8_one<<<dim3((D.f + 3) / 4, slots), 256, 0, s>>>(L, D, x, U, h);
    k_down_i8_one<<<dim3((D.d + 3) / 4, slots), 256, 0, s>>>(L, D, h, U, y);
  } else {
    k_gateup_i8<<<dim3((D.f + 3) / 4, slots), 256, 0, s>>>(L, D, x, U, h);
    k_down_i8<<<dim3((D.d + 3) / 4, slots), 256, 0, s>>>(L, D, h, U, y);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------- static scratch
// Device scratch of colimoe_route_forward_static, for callers that cannot
// allocate: a fixed array in the library's code object, one copy per device
// the library runs on, held until the process ends.  Host code never uses
// the array's name as an address (on the host it names a stand-in, not
// device memory): static_scratch_init() asks the runtime for the array's
// address on the current device once, and every launch gets that address.

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t *g_scratch_addr[kMaxDevices];  // the array's address on each device, or null
}  // namespace

hipError_t static_scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_addr[device]) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device) return hipErrorInvalidDevice;  // the device must be current
  void *ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch_addr[device] = (uint8_t *)ptr;
  return hipSuccess;
}

uint8_t *static_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch_addr[device];
}

__global__ void k_zero_words(uint32_t *__restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_zero_words(uint32_t *p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_zero_words<<<(n + 255) / 256, 256, 0, s>>>(p, n);
  return hipGetLastError();
}

}  // namespace colimoe
