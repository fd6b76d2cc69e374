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

#include "internal.h"

namespace colimoe {

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float bits_f(uint32_t v) { return __uint_as_float(v); }
__device__ __forceinline__ uint32_t f_bits(float v) { return __float_as_uint(v); }

__device__ __forceinline__ float half_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Scale of tile row `r` (0..7) from the 16-byte group record.
__device__ __forceinline__ float tile_scale(const uint4 &s, int r) {
  uint32_t w = (r >> 1) == 0 ? s.x : (r >> 1) == 1 ? s.y : (r >> 1) == 2 ? s.z : s.w;
  return (r & 1) ? half_hi(w) : half_lo(w);
}

// Dot product of 32 offset-binary nibbles (one 16-byte load) with 32 fp32
// activations, minus 8 * (their sum), which the caller passes in as `nsx`:
//   sum_i (n_i + 8 - 8) x_i = sum_i q_i x_i.
// Byte b of word i holds columns 8i+2b (low nibble) and 8i+2b+1 (high).
// Even columns accumulate into alo, odd columns (read as 16 n) into ahi.
__device__ __forceinline__ float chunk_dot(const uint4 &w, const float4 *xv, float nsx) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
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

__device__ __forceinline__ float dpp_shr(float v, int n) {
  // row_shr:n within 16-lane rows; lanes without a source read 0
  switch (n) {
    case 1: return bits_f(__builtin_amdgcn_update_dpp(0u, f_bits(v), 0x111, 0xF, 0xF, false));
    case 2: return bits_f(__builtin_amdgcn_update_dpp(0u, f_bits(v), 0x112, 0xF, 0xF, false));
    default: return bits_f(__builtin_amdgcn_update_dpp(0u, f_bits(v), 0x114, 0xF, 0xF, false));
  }
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
  const int lane = threadIdx.x & 63;
  const bool upper8 = (lane & 8) != 0;
  float keep = upper8 ? t[1] : t[0];
  float send = upper8 ? t[0] : t[1];
  float v = keep + bits_f(__builtin_amdgcn_update_dpp(0u, f_bits(send), 0x128, 0xF, 0xF, false));  // row_ror:8
  v = v + dpp_shr(v, 4);
  v = v + dpp_shr(v, 2);
  v = v + dpp_shr(v, 1);
  return v;
}

// Butterfly sum within aligned groups of `width` lanes (fixed tree).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v = v + __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

__device__ __forceinline__ int clamp_nu(const int32_t *n_unique, const Dims &D) {
  int cap = D.T * D.k < D.E ? D.T * D.k : D.E;
  int nu = D.T > 0 ? *n_unique : 0;
  return nu < 0 ? 0 : (nu > cap ? cap : nu);
}

// Work slot s of a call: routed expert ids[s] with pairs [p0, p1) for s < nu,
// else the shared expert (stored after the E routed ones) with tokens
// [0, T).  Caller-supplied union lists are clamped so no access leaves its
// buffer; an out-of-range expert id skips the slot.
__device__ __forceinline__ bool resolve_slot(const Dims &D, const UnionDev &U, int nu, int s, int &e, int &p0,
                                             int &p1) {
  if (s < nu) {
    const int tk = D.T * D.k;
    e = U.ids[s];
    p0 = U.offsets[s];
    p1 = U.offsets[s + 1];
    p0 = p0 < 0 ? 0 : (p0 > tk ? tk : p0);
    p1 = p1 < p0 ? p0 : (p1 > tk ? tk : p1);
    return e >= 0 && e < D.E;
  }
  e = D.E;
  p0 = 0;
  p1 = D.T;
  return D.n_shared > 0;
}

// ------------------------------------------------------------------- router
// A1 ([A] §1: a router picks 8 of the 256 experts): logits l[t][e] =
// sum_c R[e][c] x[t][c] + b[e] in fp32.  One wave per expert row; the row is
// held in registers and applied to every token, each token's sum taken in
// the same lane order and tree regardless of T.

template <int STEPS>
__global__ __launch_bounds__(256) void k_router_gemv(LayerDev L, Dims D, const float *__restrict__ x,
                                                     float *__restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= D.E) return;
  const float *row = L.router + (size_t)e * D.d;
  float4 r[STEPS];
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    int c = 4 * lane + 256 * i;
    r[i] = c < D.d ? *(const float4 *)(row + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float b = L.bias[e];
  for (int t = 0; t < D.T; ++t) {
    const float *xr = x + (size_t)t * D.d;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
      int c = 4 * lane + 256 * i;
      if (c < D.d) {
        float4 xv = *(const float4 *)(xr + c);
        acc = __builtin_fmaf(r[i].x, xv.x, acc);
        acc = __builtin_fmaf(r[i].y, xv.y, acc);
        acc = __builtin_fmaf(r[i].z, xv.z, acc);
        acc = __builtin_fmaf(r[i].w, xv.w, acc);
      }
    }
    acc = group_sum(acc, 64);
    if (lane == 0) logits[(size_t)t * D.E + e] = acc + b;
  }
}

// Tiled variant for many tokens: a 64x64 block of (tokens, experts), K in
// steps of 32 through LDS; each output's sum runs over c in ascending order.
__global__ __launch_bounds__(256) void k_router_gemm(LayerDev L, Dims D, const float *__restrict__ x,
                                                     float *__restrict__ logits) {
  __shared__ float xs[32][65];
  __shared__ float rs[32][65];
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < D.d; k0 += 32) {
    for (int i = threadIdx.x; i < 64 * 32; i += 256) {
      int rr = i >> 5, cc = i & 31;
      int t = t0 + rr, e = e0 + rr;
      xs[cc][rr] = t < D.T ? x[(size_t)t * D.d + k0 + cc] : 0.0f;
      rs[cc][rr] = e < D.E ? L.router[(size_t)e * D.d + k0 + cc] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = xs[kk][ty * 4 + i];
        bb[i] = rs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      int t = t0 + ty * 4 + i, e = e0 + tx * 4 + j;
      if (t < D.T && e < D.E) logits[(size_t)t * D.E + e] = acc[i][j] + L.bias[e];
    }
}

static bool launch_router_gemv(const LayerDev &L, const Dims &D, const float *x, float *logits, hipStream_t s) {
  const int steps = (D.d + 255) / 256;
  dim3 grid((D.E + 3) / 4), block(256);
#define ROUTER_CASE(S) \
  case S: k_router_gemv<S><<<grid, block, 0, s>>>(L, D, x, logits); return true;
  switch (steps) {
    ROUTER_CASE(1) ROUTER_CASE(2) ROUTER_CASE(3) ROUTER_CASE(4) ROUTER_CASE(6) ROUTER_CASE(8)
    ROUTER_CASE(12) ROUTER_CASE(16) ROUTER_CASE(24) ROUTER_CASE(32) ROUTER_CASE(48) ROUTER_CASE(64)
    default: return false;
  }
#undef ROUTER_CASE
}

hipError_t launch_router(const LayerDev &L, const Dims &D, const float *x, float *logits, hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  if (D.T <= 32 && launch_router_gemv(L, D, x, logits, s)) return hipGetLastError();
  dim3 grid((D.T + 63) / 64, (D.E + 63) / 64), block(256);
  k_router_gemm<<<grid, block, 0, s>>>(L, D, x, logits);
  return hipGetLastError();
}

// -------------------------------------------------------------------- top-k
// A2: the k largest logits, larger first, exact ties to the lower expert;
// gate weights = softmax over the selected logits.  One wave per token.

__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  uint32_t b = f_bits(v);
  if ((b & 0x7FFFFFFFu) == 0) b = 0;                       // +0 and -0 tie
  uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);  // monotone in v
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

template <int PER>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ logits, Dims D, int32_t *__restrict__ idx,
                                              float *__restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= D.T) return;
  const float *l = logits + (size_t)t * D.E;
  uint64_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int e = lane + 64 * i;
    key[i] = e < D.E ? topk_key(l[e], e) : 0ull;
  }
  float vals[16];
  int ids[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < D.k) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
      int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
      ids[j] = e;
      vals[j] = l[e];
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (key[i] == best) key[i] = 0ull;
    }
  }
  if (lane == 0) {
    const float m = vals[0];
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < D.k) sum += expf(vals[j] - m);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < D.k) {
        idx[(size_t)t * D.k + j] = ids[j];
        wout[(size_t)t * D.k + j] = expf(vals[j] - m) / sum;
      }
  }
}

hipError_t launch_topk(const float *logits, const Dims &D, int32_t *idx, float *w, hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  dim3 grid((D.T + 3) / 4), block(256);
  const int per = (D.E + 63) / 64;
  if (per <= 1)
    k_topk<1><<<grid, block, 0, s>>>(logits, D, idx, w);
  else if (per <= 2)
    k_topk<2><<<grid, block, 0, s>>>(logits, D, idx, w);
  else if (per <= 4)
    k_topk<4><<<grid, block, 0, s>>>(logits, D, idx, w);
  else if (per <= 8)
    k_topk<8><<<grid, block, 0, s>>>(logits, D, idx, w);
  else
    k_topk<16><<<grid, block, 0, s>>>(logits, D, idx, w);
  return hipGetLastError();
}

// -------------------------------------------------------------------- union
// A3 ([A] §2, batch-union: batched positions read each unique expert once):
// distinct experts ascending, and every (token, slot) pair grouped by expert
// in token order.  One wave; ranks come from per-expert lane masks, so the
// result is independent of timing.  Invalid routings (expert out of range,
// or an expert twice in one token) produce an empty union and set *err.

__global__ __launch_bounds__(64) void k_union(const int32_t *__restrict__ idx, Dims D, UnionDev U,
                                              int32_t *__restrict__ err) {
  // Dynamic LDS: masks[E] (8-byte aligned, first), counts[E], running[E], bad.
  extern __shared__ __align__(16) unsigned long long union_lds[];
  const int E = D.E, k = D.k, T = D.T;
  unsigned long long *masks = union_lds;
  int32_t *counts = (int32_t *)(union_lds + E);
  int32_t *running = counts + E;
  int32_t &bad = running[E];
  const int lane = threadIdx.x;
  if (lane == 0) bad = 0;
  for (int e = lane; e < E; e += 64) {
    counts[e] = 0;
    masks[e] = 0ull;
  }
  __syncthreads();
  for (int t = lane; t < T; t += 64) {
    for (int j = 0; j < k; ++j) {
      int e = idx[(size_t)t * k + j];
      bool ok = e >= 0 && e < E;
      for (int i = 0; i < j && ok; ++i) ok = idx[(size_t)t * k + i] != e;
      if (!ok)
        bad = 1;
      else
        atomicAdd(&counts[e], 1);
    }
  }
  __syncthreads();
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
    int a = __shfl_up(cinc, o, 64), b = __shfl_up(ninc, o, 64);
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
  __syncthreads();
  for (int t0 = 0; t0 < T; t0 += 64) {
    const int t = t0 + lane;
    const bool act = t < T;
    int ee[16];
    unsigned long long mm[16];
    int rr[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (act && j < k) {
        ee[j] = idx[(size_t)t * k + j];
        atomicOr(&masks[ee[j]], 1ull << lane);
      }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (act && j < k) {
        mm[j] = masks[ee[j]];
        rr[j] = __popcll(mm[j] & ((1ull << lane) - 1ull));
        const int p = running[ee[j]] + rr[j];
        U.pair_token[p] = t;
        U.pair_slot[p] = j;
        U.pair_of[(size_t)t * k + j] = p;
      }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (act && j < k && rr[j] == 0) {
        running[ee[j]] += __popcll(mm[j]);
        masks[ee[j]] = 0ull;
      }
    __syncthreads();
  }
}

hipError_t launch_union(const int32_t *idx, const Dims &D, const UnionDev &U, int32_t *err, hipStream_t s) {
  size_t lds = (size_t)D.E * 8 + (size_t)(2 * D.E + 1) * 4;
  k_union<<<1, 64, lds, s>>>(idx, D, U, err);
  return hipGetLastError();
}

// ----------------------------------------------------------- expert GEMVs
// A4-A6: W[r][c] = q[r][c] * s[r][c/64] ([P] "conservative correctness":
// int4, group size 64), dequantised to fp32 and multiplied in fp32 ([D] §4,
// highlight 4: at batch 1, f32 rather than integer arithmetic), fp32
// accumulation.  A wave owns one 8-row tile of one expert and streams it
// chunk by chunk (LPR lanes per row, CPL 32-column chunks per lane); each
// chunk's weights, once in registers, are applied to up to MT of the
// expert's tokens, so for calls with at most MT tokens per expert every
// weight is read from HBM once per call.  Per token and row the operations
// (chunk dots, scale fmas in chunk order, reduction tree) do not depend on MT
// or on the other tokens, which makes batched and one-at-a-time results
// bit-identical.

template <int LPR>
struct TileShape {
  static constexpr int RG = 64 / LPR;                    // row groups per wave
  static constexpr int RPG = (kTileRows + RG - 1) / RG;  // rows per lane
};

// One chunk (j) of a tile: weights + the 8 rows' scales for this lane.
template <int LPR>
__device__ __forceinline__ void load_chunk(const uint8_t *__restrict__ nib, const uint8_t *__restrict__ sc, int tile,
                                           int K, int c, uint4 (&W)[TileShape<LPR>::RPG], uint4 &S) {
  using TS = TileShape<LPR>;
  const int gr = (threadIdx.x & 63) / LPR;
  const int G = K / kGroup;
  const size_t rowb = (size_t)K / 2;
  S = *(const uint4 *)(sc + ((size_t)tile * G + (c >> 1)) * 16);
#pragma unroll
  for (int i = 0; i < TS::RPG; ++i) {
    const int r = gr + TS::RG * i;
    W[i] = r < kTileRows ? *(const uint4 *)(nib + ((size_t)tile * kTileRows + r) * rowb + (size_t)c * 16)
                         : make_uint4(0u, 0u, 0u, 0u);
  }
}

// acc[i] += s_r * (sum over the chunk of q * x) for this lane's rows.
template <int LPR>
__device__ __forceinline__ void chunk_accumulate(const uint4 (&W)[TileShape<LPR>::RPG], const uint4 &S,
                                                 const float *__restrict__ xrow, int c,
                                                 float (&acc)[TileShape<LPR>::RPG]) {
  using TS = TileShape<LPR>;
  const int gr = (threadIdx.x & 63) / LPR;
  float4 xv[8];
  const float4 *src = (const float4 *)(xrow + (size_t)kChunk * c);
#pragma unroll
  for (int v = 0; v < 8; ++v) xv[v] = src[v];
  const float nsx = neg8_sum(xv);
#pragma unroll
  for (int i = 0; i < TS::RPG; ++i) {
    const int r = gr + TS::RG * i;
    if (r < kTileRows) acc[i] = __builtin_fmaf(tile_scale(S, r), chunk_dot(W[i], xv, nsx), acc[i]);
  }
}

// Reduce a tile for one token.  LPR == 64: lane 8r+7 returns row r's sum.
// Otherwise the 8 row sums go to `rows` (wave-private LDS).
template <int LPR>
__device__ __forceinline__ float tile_reduce(const float *acc, float *rows) {
  using TS = TileShape<LPR>;
  if constexpr (LPR == 64) {
    return reduce8_rows(acc);
  } else {
    const int lane = threadIdx.x & 63;
    const int q = lane % LPR, gr = lane / LPR;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < TS::RPG; ++i) {
      const float v = group_sum(acc[i], LPR);
      const int r = gr + TS::RG * i;
      if (q == 0 && r < kTileRows) rows[r] = v;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return 0.0f;
  }
}

// Accumulate one tile over all K for up to MT tokens (token i of the group is
// pair p0 + i of the slot).  acc[m][i]: lane partial of row i for token m.
template <int LPR, int CPL, int MT>
__device__ __forceinline__ void tile_pass(const uint8_t *__restrict__ nib, const uint8_t *__restrict__ sc, int tile,
                                          int K, const float *__restrict__ xbase, size_t xstride,
                                          const int (&xrow)[MT], int mcount, float (&acc)[MT][TileShape<LPR>::RPG]) {
  using TS = TileShape<LPR>;
  const int q = (threadIdx.x & 63) % LPR;
  const int C = K / kChunk;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < TS::RPG; ++i) acc[m][i] = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = q + LPR * j;
    if (c < C) {
      uint4 W[TS::RPG], S;
      load_chunk<LPR>(nib, sc, tile, K, c, W, S);
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < mcount) chunk_accumulate<LPR>(W, S, xbase + (size_t)xrow[m] * xstride, c, acc[m]);
    }
  }
}

// Token p of slot s: its activation row and output row.
__device__ __forceinline__ void slot_token(const Dims &D, const UnionDev &U, int nu, int s, int p, int &t, int &orow) {
  if (s < nu) {
    t = U.pair_token[p];
    orow = p;
  } else {
    t = p;
    orow = D.T * D.k + p;
  }
}

// Gate/up for every (unique expert, tile of 4 gate + 4 up rows) item, applied
// to each of the expert's tokens: h = SiLU(g) * u, written per pair.  Slot nu
// (after the routed experts) is the shared expert with all T tokens ([D] §3).
template <int LPR, int CPL, int MT>
__global__ __launch_bounds__(256) void k_gateup(LayerDev L, Dims D, const float *__restrict__ x, UnionDev U,
                                                float *__restrict__ h, float *__restrict__ gdbg,
                                                float *__restrict__ udbg) {
  using TS = TileShape<LPR>;
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
    const uint8_t *base = L.experts + (size_t)e * L.expert_stride;
    for (int pg = p0; pg < p1; pg += MT) {
      const int mcount = min(MT, p1 - pg);
      int xrow[MT], orows[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        int t = 0, orow = -1;
        if (m < mcount) slot_token(D, U, nu, s, pg + m, t, orow);
        if (t < 0 || t >= D.T) {
          t = 0;
          orow = -1;
        }
        xrow[m] = t;
        orows[m] = orow;
      }
      float acc[MT][TS::RPG];
      tile_pass<LPR, CPL, MT>(base + EL.gu_nib, base + EL.gu_sc, ti, D.d, x, (size_t)D.d, xrow, mcount, acc);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < mcount) {
          const float v = tile_reduce<LPR>(acc[m], rows_lds[wave]);
          float g, u;
          int r;
          bool writer;
          if constexpr (LPR == 64) {
            auto sw = __builtin_amdgcn_permlane32_swap(f_bits(v), f_bits(v), false, false);
            u = bits_f(sw[1]);  // lanes < 32 receive lane + 32
            g = v;
            r = lane >> 3;
            writer = (lane & 7) == 7 && r < 4;
          } else {
            r = lane & 3;
            writer = lane < 4;
            g = rows_lds[wave][r];
            u = rows_lds[wave][r + 4];
          }
          if (writer && orows[m] >= 0) {
            const size_t o = (size_t)orows[m] * D.f + (size_t)ti * 4 + r;
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
}

// Down projection y = Wd h for every (unique expert, 8-row tile) item and
// each of the expert's tokens, written per pair (shared: row T*k + t).
template <int LPR, int CPL, int MT>
__global__ __launch_bounds__(256) void k_down(LayerDev L, Dims D, const float *__restrict__ h, UnionDev U,
                                              float *__restrict__ y) {
  using TS = TileShape<LPR>;
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
    const uint8_t *base = L.experts + (size_t)e * L.expert_stride;
    for (int pg = p0; pg < p1; pg += MT) {
      const int mcount = min(MT, p1 - pg);
      int orows[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) orows[m] = m < mcount ? ((s < nu) ? pg + m : D.T * D.k + pg + m) : 0;
      float acc[MT][TS::RPG];
      tile_pass<LPR, CPL, MT>(base + EL.dn_nib, base + EL.dn_sc, ti, D.f, h, (size_t)D.f, orows, mcount, acc);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < mcount) {
          float v = tile_reduce<LPR>(acc[m], rows_lds[wave]);
          int r;
          bool writer;
          if constexpr (LPR == 64) {
            r = lane >> 3;
            writer = (lane & 7) == 7;
          } else {
            r = lane & 7;
            writer = lane < kTileRows;
            v = rows_lds[wave][r];
          }
          if (writer) y[(size_t)orows[m] * D.d + (size_t)ti * kTileRows + r] = v;
        }
      }
    }
  }
}

struct GemvGrid {
  dim3 grid, block;
};

static GemvGrid gemv_grid(int items_max) {
  int blocks = (items_max + 3) / 4;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  return {dim3(blocks), dim3(256)};
}

// Lane shape from K (the matrix's input length): 64 lanes per row with CPL
// chunks each when K >= 2048, else one chunk per lane and 64/LPR rows side
// by side.  MT: tokens per pass, 1 when no expert can have more than one
// token (T == 1), else 16.
#define GEMV_LAUNCH(KERNEL, LPR_, CPL_, ...)                                             \
  do {                                                                                   \
    if (mt1)                                                                             \
      KERNEL<LPR_, CPL_, 1><<<G.grid, G.block, 0, s>>>(__VA_ARGS__);                     \
    else                                                                                 \
      KERNEL<LPR_, CPL_, 16><<<G.grid, G.block, 0, s>>>(__VA_ARGS__);                    \
  } while (0)

#define GEMV_DISPATCH(KERNEL, K, ...)                                          \
  do {                                                                         \
    const int C_ = (K) / kChunk;                                               \
    if (C_ >= 64) {                                                            \
      switch ((C_ + 63) / 64) {                                                \
        case 1: GEMV_LAUNCH(KERNEL, 64, 1, __VA_ARGS__); break;                \
        case 2: GEMV_LAUNCH(KERNEL, 64, 2, __VA_ARGS__); break;                \
        case 3: GEMV_LAUNCH(KERNEL, 64, 3, __VA_ARGS__); break;                \
        case 4: GEMV_LAUNCH(KERNEL, 64, 4, __VA_ARGS__); break;                \
        case 5: GEMV_LAUNCH(KERNEL, 64, 5, __VA_ARGS__); break;                \
        case 6: GEMV_LAUNCH(KERNEL, 64, 6, __VA_ARGS__); break;                \
        case 7: GEMV_LAUNCH(KERNEL, 64, 7, __VA_ARGS__); break;                \
        case 8: GEMV_LAUNCH(KERNEL, 64, 8, __VA_ARGS__); break;                \
        default: return hipErrorInvalidValue;                                  \
      }                                                                        \
    } else if (C_ > 16) {                                                      \
      GEMV_LAUNCH(KERNEL, 32, 1, __VA_ARGS__);                                 \
    } else if (C_ > 8) {                                                       \
      GEMV_LAUNCH(KERNEL, 16, 1, __VA_ARGS__);                                 \
    } else if (C_ > 4) {                                                       \
      GEMV_LAUNCH(KERNEL, 8, 1, __VA_ARGS__);                                  \
    } else if (C_ > 2) {                                                       \
      GEMV_LAUNCH(KERNEL, 4, 1, __VA_ARGS__);                                  \
    } else {                                                                   \
      GEMV_LAUNCH(KERNEL, 2, 1, __VA_ARGS__);                                  \
    }                                                                          \
  } while (0)

static int slots_max(const Dims &D) {
  long long tk = (long long)D.T * D.k;
  return (int)(tk < D.E ? tk : D.E) + D.n_shared;
}

hipError_t launch_gateup(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h,
                         hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  const bool mt1 = D.T == 1;
  GemvGrid G = gemv_grid(slots_max(D) * (D.f / 4));
  GEMV_DISPATCH(k_gateup, D.d, L, D, x, U, h, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_down(const LayerDev &L, const Dims &D, const float *h, const UnionDev &U, float *y,
                       hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  const bool mt1 = D.T == 1;
  GemvGrid G = gemv_grid(slots_max(D) * (D.d / kTileRows));
  GEMV_DISPATCH(k_down, D.f, L, D, h, U, y);
  return hipGetLastError();
}

// ------------------------------------------------------------------ combine
// A7: r[t] += sum over the token's experts in ascending id of w * y, then the
// shared expert's y (weight 1).  Fixed order, no atomics: a token's result
// is the same whether it runs alone or batched.

__global__ __launch_bounds__(256) void k_combine(Dims D, const int32_t *__restrict__ idx,
                                                 const float *__restrict__ w, UnionDev U,
                                                 const float *__restrict__ y, float *__restrict__ residual) {
  const int t = blockIdx.y;
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (t >= D.T || r >= D.d) return;
  // A token's pairs sit in ascending expert order in the union lists, so
  // visiting its slots by increasing pair index visits experts ascending.
  const int nu = clamp_nu(U.n_unique, D);
  const int tk = D.T * D.k;
  float acc = residual[(size_t)t * D.d + r];
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
        if (best < tk) acc = __builtin_fmaf(w[(size_t)t * D.k + bj], y[(size_t)best * D.d + r], acc);
        prev = best;
      }
    }
  }
  if (D.n_shared) acc = acc + y[((size_t)D.T * D.k + t) * D.d + r];
  residual[(size_t)t * D.d + r] = acc;
}

hipError_t launch_combine(const Dims &D, const int32_t *idx, const float *w, const UnionDev &U, const float *y,
                          float *residual, hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  dim3 grid((D.d + 255) / 256, D.T), block(256);
  k_combine<<<grid, block, 0, s>>>(D, idx, w, U, y, residual);
  return hipGetLastError();
}

// ------------------------------------------------------------------ rmsnorm
// x = r / sqrt(mean(r^2) + eps), unit weight; one block per token, fixed
// reduction order.

__global__ __launch_bounds__(256) void k_rmsnorm(const float *__restrict__ r, int d, float eps,
                                                 float *__restrict__ x) {
  __shared__ float part[4];
  const int t = blockIdx.x;
  const float *rr = r + (size_t)t * d;
  float acc = 0.0f;
  for (int c = threadIdx.x; c < d; c += 256) acc = __builtin_fmaf(rr[c], rr[c], acc);
  acc = group_sum(acc, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  const float ss = (part[0] + part[1]) + (part[2] + part[3]);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  for (int c = threadIdx.x; c < d; c += 256) x[(size_t)t * d + c] = rr[c] * inv;
}

hipError_t launch_rmsnorm(const float *r, int T, int d, float eps, float *x, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  k_rmsnorm<<<T, 256, 0, s>>>(r, d, eps, x);
  return hipGetLastError();
}

// --------------------------------------------------------------- debug path
// One expert, one token, through the same kernels (a one-slot union that the
// caller wrote into the workspace).

hipError_t launch_debug_gateup(const LayerDev &L, const Dims &D, const float *x, const UnionDev &U, float *h,
                               float *g, float *u, hipStream_t s) {
  const bool mt1 = true;
  GemvGrid G = gemv_grid(D.f / 4);
  GEMV_DISPATCH(k_gateup, D.d, L, D, x, U, h, g, u);
  return hipGetLastError();
}

}  // namespace colimoe
