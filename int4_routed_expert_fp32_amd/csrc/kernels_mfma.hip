// kernels_mfma.hip - bf16 MFMA path of the MoE layer for prefill-shaped calls
// (many tokens per expert), gfx950 (CDNA4).
//
// Pages cited by title and section:
//   [A] "Colibrì: running a 744B MoE model on a laptop with 2400 lines of pure C"
//       (kechuai.cn article)
//   [D] "colibrì: 1300 lines of C, a 25 GB laptop, a 744-billion-parameter model"
//       (SSP GitHub Daily #091, jsqmd.com)
//
// What is computed ([A] §2: the experts picked for a batch are read once and
// applied to every token routed to them; [D] §4, highlight 4: the int4 kernel
// pays off once it works on a batch): the tokens of a call are grouped by
// expert (the union lists), every group is an M x K by K x N product against
// the expert's weights, dequantised to bf16 as bf16(q * s) with
// round-to-nearest-even, activations rounded to bf16 the same way, fp32
// accumulation on the matrix cores; SiLU(gate) * up in fp32 rounded to bf16
// feeds the down product, whose fp32 rows go to the combine kernel.
//
// Work decomposition.  An M-block is up to kMB = 128 consecutive rows (pairs)
// of one expert; an item is (M-block, kNT = 256 weight rows), taken by a block
// of 4 waves with v_mfma_f32_32x32x16_bf16 (32 x 32 outputs, K = 16).  Lane
// (j, hh) (j = lane % 32, hh = lane / 32) dequantises chunk 2g + hh of its
// weight row for group g: the 4 words are the B operands of the group's 4
// MFMAs, and A is read with the same K order inside the group (16 bytes of an
// activation row at column 64g + 32hh + 8q for MFMA q).  Items are taken in
// rounds; inside a round the 8 XCDs get contiguous ranges so that the weight
// tiles of one M-block run on one XCD and share its L2 for the activation rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace colimoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 of an fp32 value, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// v_and_or_b32 (x & mask) | magic, mask in a scalar register (one constant
// per VOP3 instruction on gfx9).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(magic));
  return r;
}

__device__ __forceinline__ float half_lo_f(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
}
__device__ __forceinline__ float half_hi_f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(h >> 16)); }

// Scale constants of one weight group for dequant8.
struct GroupScale {
  float s, m1032, s16, m72;
  __device__ __forceinline__ explicit GroupScale(float sc)
      : s(sc), m1032(-1032.0f * sc), s16(0.0625f * sc), m72(-72.0f * sc) {}
};

// 8 int4 weights (one word of two's-complement nibbles, element 2b in the low
// nibble of byte b) times their group scale s, rounded to bf16.  Each word is
// flipped to offset binary n = q + 8; nibbles are dropped into the mantissas of
// fp16 halves with exponent 10 (0x6400 = 1024): bits 0-3 give 1024 + n, bits
// 4-7 give 1024 + 16 n.  One v_fma_mix_f32 per weight then forms
// (1024 + n) s - 1032 s, or (1024 + 16 n) (s/16) - 72 s, both exactly
// (n - 8) s = q s in fp32 (at most 15 significant bits), and v_cvt_pk_bf16_f32
// rounds pairs to bf16, to nearest even.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, const GroupScale &g, uint32_t magic) {
  const uint32_t x = w ^ 0x88888888u, y = x >> 8;
  const uint32_t h0 = and_or(x, 0x000F000Fu, magic);  // elements 0, 4
  const uint32_t h1 = and_or(x, 0x00F000F0u, magic);  // elements 1, 5 (times 16)
  const uint32_t h2 = and_or(y, 0x000F000Fu, magic);  // elements 2, 6
  const uint32_t h3 = and_or(y, 0x00F000F0u, magic);  // elements 3, 7 (times 16)
  bf16x8 r;
  r[0] = (__bf16)__builtin_fmaf(half_lo_f(h0), g.s, g.m1032);
  r[1] = (__bf16)__builtin_fmaf(half_lo_f(h1), g.s16, g.m72);
  r[2] = (__bf16)__builtin_fmaf(half_lo_f(h2), g.s, g.m1032);
  r[3] = (__bf16)__builtin_fmaf(half_lo_f(h3), g.s16, g.m72);
  r[4] = (__bf16)__builtin_fmaf(half_hi_f(h0), g.s, g.m1032);
  r[5] = (__bf16)__builtin_fmaf(half_hi_f(h1), g.s16, g.m72);
  r[6] = (__bf16)__builtin_fmaf(half_hi_f(h2), g.s, g.m1032);
  r[7] = (__bf16)__builtin_fmaf(half_hi_f(h3), g.s16, g.m72);
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

// ------------------------------------------------------------- M-block list
// One wave: for each slot (unique routed expert in union order, then the
// shared expert) its rows split into M-blocks of kMB; entries (expert, first
// row, rows).  Rows of routed slots are pair positions, those of the shared
// expert are T*k + token.  M-blocks of at most 32 rows (one M-tile: most
// experts of a prefill call, and the last block of a large one) go to
// list[0..count[0]), the others to list[max_entries..max_entries+count[1]):
// each class runs in a GEMM kernel sized for it.
__global__ __launch_bounds__(64) void k_mblocks(Dims D, UnionDev U, int4 *__restrict__ list,
                                                int32_t *__restrict__ count, int max_entries) {
  const int lane = threadIdx.x;
  const int nu = clamp_nu(U.n_unique, D);
  const int slots = nu + (D.n_shared > 0 ? 1 : 0);
  int run_s = 0, run_l = 0;
  for (int base = 0; base < slots; base += 64) {
    const int s = base + lane;
    int e = 0, p0 = 0, p1 = 0, cnt = 0, row0 = 0;
    if (s < slots && resolve_slot(D, U, nu, s, e, p0, p1)) {
      row0 = s < nu ? p0 : D.T * D.k;
      cnt = (p1 - p0 + kMB - 1) / kMB;
    }
    // only the last M-block of a slot can hold 32 rows or fewer
    const int last_rows = cnt > 0 ? p1 - p0 - (cnt - 1) * kMB : 0;
    const int ns = (cnt > 0 && last_rows <= 32) ? 1 : 0, nl = cnt - ns;
    int is = ns, il = nl;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int vs = __shfl_up(is, o, 64), vl = __shfl_up(il, o, 64);
      if (lane >= o) {
        is += vs;
        il += vl;
      }
    }
    const int ps = run_s + is - ns, pl = run_l + il - nl;
    for (int b = 0; b < nl; ++b)
      if (pl + b < max_entries)
        list[max_entries + pl + b] = make_int4(e, row0 + b * kMB, min(kMB, p1 - p0 - b * kMB), 0);
    if (ns && ps < max_entries) list[ps] = make_int4(e, row0 + nl * kMB, last_rows, 0);
    run_s += __shfl(is, 63, 64);
    run_l += __shfl(il, 63, 64);
  }
  if (lane == 0) {
    count[0] = run_s < max_entries ? run_s : max_entries;
    count[1] = run_l < max_entries ? run_l : max_entries;
  }
}

// ---------------------------------------------------- activations in bf16
// Row t of xb = bf16(x[t]), one row per token; the gate/up GEMM reads a
// pair's row through the pair's token (the union lists' pair_token; rows
// T*k + t of the shared expert are token t).
__global__ __launch_bounds__(256) void k_gather_bf16(const float *__restrict__ x, Dims D,
                                                     uint16_t *__restrict__ xb) {
  for (int t = blockIdx.x; t < D.T; t += gridDim.x) {
    const float *src = x + (size_t)t * D.d;
    uint16_t *dst = xb + (size_t)t * D.d;
    for (int c = 8 * threadIdx.x; c < D.d; c += 8 * 256) {
      const float4 a = *(const float4 *)(src + c), b = *(const float4 *)(src + c + 4);
      uint4 o;
      o.x = (uint32_t)bf16_bits(a.x) | ((uint32_t)bf16_bits(a.y) << 16);
      o.y = (uint32_t)bf16_bits(a.z) | ((uint32_t)bf16_bits(a.w) << 16);
      o.z = (uint32_t)bf16_bits(b.x) | ((uint32_t)bf16_bits(b.y) << 16);
      o.w = (uint32_t)bf16_bits(b.z) | ((uint32_t)bf16_bits(b.w) << 16);
      *(uint4 *)(dst + c) = o;
    }
  }
}

// ------------------------------------------------------------ grouped GEMM
// GATEUP: A = xb [rows][d], weights = interleaved gate/up rows (2f of them),
//         output hb [rows][f] = bf16(SiLU(g) * u).
// down:   A = hb [rows][f], weights = down rows (d of them), output y [rows][d]
//         fp32.
// Block: 4 waves, item = (M-block of up to 128 rows, 256 weight rows); wave w
// owns weight rows 64w..64w+63 of the item as two 32-column MFMA tiles, so
// each A operand read from LDS feeds two MFMAs.  Per 64-wide K group the
// block stages the M-block's A tile (128 rows x 128 bytes, rows padded to 144
// bytes so the 16-byte reads of 16 consecutive lanes hit distinct banks) in
// one of two LDS buffers while the other is consumed.  Loads run two groups
// ahead (A into one of two register sets, weights and scales likewise), and
// the barrier between groups waits only for LDS traffic, so loads stay in
// flight across it.
constexpr int kArowBytes = 144;

// Barrier for the LDS ring: LDS writes of this wave complete, then s_barrier;
// vector-memory loads issued earlier stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
  __builtin_amdgcn_s_barrier();
}

// 16 NP bytes of one A row staged in registers between its load and its LDS
// store.  Loader threads past the M-block's last row read the block's first
// row instead: output row i of an MFMA depends only on A row i, and rows past
// the block are never stored.
template <int NP>  // 16-byte pieces per thread: NMT (rows 32 NMT x 128 bytes over 256 threads)
struct AStage {
  u32x4 a[NP];
  __device__ __forceinline__ void load(const u32x4 *src) {
#pragma unroll
    for (int i = 0; i < NP; ++i) a[i] = src[i];
  }
  __device__ __forceinline__ void store(unsigned char *dst) const {
#pragma unroll
    for (int i = 0; i < NP; ++i) *(u32x4 *)(dst + 16 * i) = a[i];
  }
};

struct WStage {
  u32x4 w0, w1;  // chunk of weight rows gr0 and gr0 + 32
  float s0, s1;  // their group scales
};

template <bool GATEUP>
struct GemmItem {
  const uint8_t *nib;
  const uint16_t *sc0, *sc1;
  int tile0, tile1, r, K;
  bool wact;
  __device__ __forceinline__ void load(int g, WStage &st) const {
    st.w0 = *(const u32x4 *)(nib + chunk_offset(tile0, K, 2 * g + (threadIdx.x >> 5 & 1), r));
    st.w1 = *(const u32x4 *)(nib + chunk_offset(tile1, K, 2 * g + (threadIdx.x >> 5 & 1), r));
    st.s0 = (float)__builtin_bit_cast(_Float16, sc0[(size_t)g * 8]);
    st.s1 = (float)__builtin_bit_cast(_Float16, sc1[(size_t)g * 8]);
  }
};

// One K group: dequantise the lane's two weight chunks and run the MFMAs of
// the M-tiles that hold rows.  Done in two halves of K (MFMAs 0-1, then 2-3)
// so only half of the B and A operands are live at a time.
template <int NMT_MAX>
__device__ __forceinline__ void gemm_group(const unsigned char *cur, const WStage &st, int nmt, int j, int hh,
                                           f32x16 (&acc)[NMT_MAX][2]) {
  const GroupScale g0(st.s0), g1(st.s1);
  const uint32_t magic = 0x64006400u;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const bf16x8 b00 = dequant8(st.w0[2 * half], g0, magic);
    const bf16x8 b01 = dequant8(st.w0[2 * half + 1], g0, magic);
    const bf16x8 b10 = dequant8(st.w1[2 * half], g1, magic);
    const bf16x8 b11 = dequant8(st.w1[2 * half + 1], g1, magic);
#pragma unroll
    for (int mt = 0; mt < NMT_MAX; ++mt) {
      if (mt < nmt) {
        const unsigned char *ar = cur + (32 * mt + j) * kArowBytes + 64 * hh + 32 * half;
        const u32x4 a0 = *(const u32x4 *)(ar), a1 = *(const u32x4 *)(ar + 16);
        acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), b00, acc[mt][0], 0, 0, 0);
        acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), b10, acc[mt][1], 0, 0, 0);
        acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a1), b01, acc[mt][0], 0, 0, 0);
        acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a1), b11, acc[mt][1], 0, 0, 0);
      }
    }
  }
}

template <bool GATEUP, int NMT>
__global__ __launch_bounds__(256, NMT == 1 ? 3 : 2) void k_gemm_mfma(LayerDev L, Dims D, const uint16_t *__restrict__ A,
                                                      const int32_t *__restrict__ pair_token,
                                                      const int4 *__restrict__ list,
                                                      const int32_t *__restrict__ count, int max_entries,
                                                      uint16_t *__restrict__ hb, float *__restrict__ y) {
  constexpr int kRows = 32 * NMT;              // rows of an M-block this kernel takes
  constexpr int kBuf = kRows * kArowBytes;     // bytes of one A stage
  constexpr int kTPR = 8 / NMT;                // loader threads per A row (16 NMT bytes each)
  __shared__ __align__(16) unsigned char As[2 * kBuf];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, hh = lane >> 5;
  const int K = GATEUP ? D.d : D.f;
  const int nrows = GATEUP ? 2 * D.f : D.d;
  const int ntiles = (nrows + kNT - 1) / kNT;
  const int G = K / kGroup;
  const ExpertLayout EL = expert_layout(D.d, D.f);
  int nmb = *count;
  nmb = nmb < 0 ? 0 : (nmb > max_entries ? max_entries : nmb);
  const int items = nmb * ntiles;
  const int per_xcd = gridDim.x >> 3;  // gridDim.x is a multiple of 8
  const int slot_in_round = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  // A loader role of this thread: row t/kTPR, bytes 16 NMT (t % kTPR) .. of the group
  const int lrow = threadIdx.x / kTPR, lpart = threadIdx.x % kTPR;
  for (int base = 0; base < items; base += gridDim.x) {
    const int item = base + slot_in_round;
    if (item >= items) continue;  // block-uniform
    const int mb = item / ntiles, nt = item - mb * ntiles;
    const int4 ent = list[mb];
    const int e = ent.x, row0 = ent.y, rc = ent.z;
    const int nmt = (rc + 31) >> 5;  // M-tiles holding rows (1..NMT)
    GemmItem<GATEUP> it;
    // weight rows come in multiples of 64; a wave past the last one computes
    // on row 0's weights (valid memory) and stores nothing
    it.wact = nt * kNT + 64 * wave < nrows;
    const int gr0 = it.wact ? nt * kNT + 64 * wave + j : j;
    it.tile0 = gr0 >> 3;
    it.tile1 = (gr0 + 32) >> 3;
    it.r = gr0 & 7;
    it.K = K;
    const uint8_t *base_e = expert_base(L, e);
    it.nib = base_e + (GATEUP ? EL.gu_nib : EL.dn_nib);
    const uint16_t *scb = (const uint16_t *)(base_e + (GATEUP ? EL.gu_sc : EL.dn_sc));
    it.sc0 = scb + (size_t)it.tile0 * G * 8 + it.r;
    it.sc1 = scb + (size_t)it.tile1 * G * 8 + it.r;
    const bool lok = lrow < rc;
    int arow = row0 + (lok ? lrow : 0);
    if (GATEUP) {  // A = x in bf16, one row per token: the row's token
      const int tk = D.T * D.k;
      arow = arow < tk ? pair_token[arow] : arow - tk;
      arow = arow >= 0 && arow < D.T ? arow : 0;  // a row of caller-supplied lists' bad token: never combined
    }
    const u32x4 *asrc = (const u32x4 *)(A + (size_t)arow * K + 8 * NMT * lpart);
    unsigned char *adst = As + lrow * kArowBytes + 16 * NMT * lpart;

    f32x16 acc[NMT][2];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mt][n][v] = 0.0f;

    // Prologue: A(0) into LDS buffer 0; A(1), W(0) and W(1) in flight.  The
    // loop below loads unconditionally (group indices clamped to G - 1, a
    // redundant but valid load at the tail) so the compiler can count
    // outstanding loads exactly and wait only for the ones it consumes.
    const int G1 = G - 1;
    AStage<NMT> rA, rB;
    rA.load(asrc);
    rA.store(adst);
    rB.load(asrc + 8 * min(1, G1));
    WStage sE, sO;
    it.load(0, sE);
    it.load(min(1, G1), sO);
    lds_barrier();
    // groups in pairs: even groups use LDS buffer 0 and register sets rA / sE
    for (int g = 0; g < G; g += 2) {
      // ---- even group g: A(g+1) is in rB, A(g+2) goes to rA
      rA.load(asrc + 8 * min(g + 2, G1));
      gemm_group<NMT>(As, sE, nmt, j, hh, acc);
      it.load(min(g + 2, G1), sE);
      rB.store(adst + kBuf);
      lds_barrier();
      if (g + 1 >= G) break;
      // ---- odd group g+1: A(g+2) is in rA, A(g+3) goes to rB
      rB.load(asrc + 8 * min(g + 3, G1));
      gemm_group<NMT>(As + kBuf, sO, nmt, j, hh, acc);
      it.load(min(g + 3, G1), sO);
      rA.store(adst);
      lds_barrier();
    }

    // Epilogue.  Accumulator element v of lane (j, hh) is row 8(v/4) + 4hh + v%4
    // of the M-tile, column j of the 32-column tile.
    if (it.wact) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        if (mt < nmt) {
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            const int gr = gr0 + 32 * n;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int rr = 32 * mt + 8 * (v >> 2) + 4 * hh + (v & 3);
              const float val = acc[mt][n][v];
              if (GATEUP) {
                // tile rows 0-3 are gate rows, 4-7 the up rows of the same features
                const float up = __shfl_down(val, 4, 64);
                if ((j & 7) < 4 && rr < rc) {
                  const int feat = 4 * (gr >> 3) + (j & 3);
                  hb[(size_t)(row0 + rr) * D.f + feat] = bf16_bits(silu_f(val) * up);
                }
              } else {
                if (rr < rc) y[(size_t)(row0 + rr) * D.d + gr] = val;
              }
            }
          }
        }
      }
    }
  }
}

// ----------------------------------------------------- router, many tokens
// A1 for many tokens: logits = x R^T + b in fp32 on the matrix cores
// (v_mfma_f32_32x32x2_f32).  Block: 64 tokens x 64 experts over one of S
// K-slices of d (4 waves, 32 x 32 each), K staged in LDS 32 columns at a
// time; slices write fp32 partials that k_router_reduce sums in slice order
// and adds the bias to.  A logit depends only on its token's row, so the
// result does not depend on which other tokens share the call.
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void k_router_mfma(LayerDev L, Dims D, const float *__restrict__ x,
                                                     float *__restrict__ part, int S) {
  __shared__ float xs[64][33];
  __shared__ float rs[64][33];
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64, ks = blockIdx.z;
  const int Kc = D.d / S, kbeg = ks * Kc;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wt = wave >> 1, we = wave & 1, i = lane & 31, kh = lane >> 5;
  const int lr = threadIdx.x >> 2, lc = (threadIdx.x & 3) * 8;  // loader: row, first of 8 columns
  const int lt = t0 + lr, le = e0 + lr;
  const float *xrow = x + (size_t)(lt < D.T ? lt : 0) * D.d;
  const float *rrow = L.router + (size_t)(le < D.E ? le : 0) * D.d;
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  for (int k0 = kbeg; k0 < kbeg + Kc; k0 += 32) {
    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0, r0 = x0, r1 = x0;
    if (lt < D.T) {
      x0 = *(const float4 *)(xrow + k0 + lc);
      x1 = *(const float4 *)(xrow + k0 + lc + 4);
    }
    if (le < D.E) {
      r0 = *(const float4 *)(rrow + k0 + lc);
      r1 = *(const float4 *)(rrow + k0 + lc + 4);
    }
    float *xd = &xs[lr][lc], *rd = &rs[lr][lc];
    xd[0] = x0.x; xd[1] = x0.y; xd[2] = x0.z; xd[3] = x0.w;
    xd[4] = x1.x; xd[5] = x1.y; xd[6] = x1.z; xd[7] = x1.w;
    rd[0] = r0.x; rd[1] = r0.y; rd[2] = r0.z; rd[3] = r0.w;
    rd[4] = r1.x; rd[5] = r1.y; rd[6] = r1.z; rd[7] = r1.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(xs[32 * wt + i][2 * kk + kh], rs[32 * we + i][2 * kk + kh], acc, 0, 0,
                                                0);
    __syncthreads();
  }
  // element v of lane (i, kh): token row 8(v/4) + 4kh + v%4 of the wave tile, expert column i
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int tt = t0 + 32 * wt + 8 * (v >> 2) + 4 * kh + (v & 3), ee = e0 + 32 * we + i;
    if (tt < D.T && ee < D.E) part[((size_t)ks * D.T + tt) * D.E + ee] = acc[v];
  }
}

__global__ __launch_bounds__(256) void k_router_reduce(const float *__restrict__ part, int S, LayerDev L, Dims D,
                                                       float *__restrict__ logits) {
  const size_t n = (size_t)D.T * D.E;
  for (size_t o = (size_t)blockIdx.x * 256 + threadIdx.x; o < n; o += (size_t)gridDim.x * 256) {
    float sum = part[o];
    for (int ks = 1; ks < S; ++ks) sum = sum + part[(size_t)ks * n + o];
    logits[o] = sum + L.bias[o % D.E];
  }
}

// ---------------------------------------------------------------- launchers

int router_splits(int d) {
  for (int S = 8; S > 1; S >>= 1)
    if (d % (32 * S) == 0) return S;
  return 1;
}

hipError_t launch_router_mfma(const LayerDev &L, const Dims &D, const float *x, float *part, float *logits,
                              hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  const int S = router_splits(D.d);
  dim3 g((D.T + 63) / 64, (D.E + 63) / 64, S);
  k_router_mfma<<<g, 256, 0, s>>>(L, D, x, part, S);
  const size_t n = (size_t)D.T * D.E;
  k_router_reduce<<<(int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096), 256, 0, s>>>(part, S, L, D, logits);
  return hipGetLastError();
}


int mfma_max_entries(int T, int k, int E, int n_shared) {
  const int tk = T * k;
  const int ue = tk < E ? tk : E;
  return (tk + kMB - 1) / kMB + ue + (n_shared > 0 ? (T + kMB - 1) / kMB : 0) + 1;
}

hipError_t launch_mblocks(const Dims &D, const UnionDev &U, int4 *list, int32_t *count, int max_entries,
                          hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  k_mblocks<<<1, 64, 0, s>>>(D, U, list, count, max_entries);
  return hipGetLastError();
}

hipError_t launch_gather_bf16(const float *x, const Dims &D, uint16_t *xb, hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  k_gather_bf16<<<D.T < 8192 ? D.T : 8192, 256, 0, s>>>(x, D, xb);
  return hipGetLastError();
}

// Blocks of the persistent grid: a multiple of 8 (one share per XCD), `per_cu`
// blocks per CU.
static int mfma_grid(int max_entries, int ntiles, int per_cu) {
  const long items = (long)max_entries * ntiles;
  long g = 256L * per_cu;
  if (items < g) g = (items + 7) / 8 * 8;
  return (int)(g < 8 ? 8 : g);
}

// M-blocks of one M-tile (list[0..count[0])) and of up to four
// (list[max_entries..], count[1]), one kernel each.
hipError_t launch_gateup_mfma(const LayerDev &L, const Dims &D, const uint16_t *xb, const UnionDev &U,
                              const int4 *list, const int32_t *count, int max_entries, uint16_t *hb, hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  const int ntiles = (2 * D.f + kNT - 1) / kNT;
  k_gemm_mfma<true, 1><<<mfma_grid(max_entries, ntiles, 3), 256, 0, s>>>(L, D, xb, U.pair_token, list, count,
                                                                          max_entries, hb, nullptr);
  k_gemm_mfma<true, 4><<<mfma_grid(max_entries, ntiles, 2), 256, 0, s>>>(L, D, xb, U.pair_token, list + max_entries,
                                                                          count + 1, max_entries, hb, nullptr);
  return hipGetLastError();
}

hipError_t launch_down_mfma(const LayerDev &L, const Dims &D, const uint16_t *hb, const int4 *list,
                            const int32_t *count, int max_entries, float *y, hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  const int ntiles = (D.d + kNT - 1) / kNT;
  k_gemm_mfma<false, 1><<<mfma_grid(max_entries, ntiles, 3), 256, 0, s>>>(L, D, hb, nullptr, list, count,
                                                                           max_entries, nullptr, y);
  k_gemm_mfma<false, 4><<<mfma_grid(max_entries, ntiles, 2), 256, 0, s>>>(L, D, hb, nullptr, list + max_entries,
                                                                           count + 1, max_entries, nullptr, y);
  return hipGetLastError();
}

}  // namespace colimoe
