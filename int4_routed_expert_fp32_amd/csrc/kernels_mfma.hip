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
// of one expert; an item is (M-block, 128 weight rows).  A block of 4 waves
// takes an item; wave w owns 32 weight rows and all M-tiles (32 rows each) of
// the M-block that hold rows, with v_mfma_f32_32x32x16_bf16.  Lane (j, hh)
// (j = lane % 32, hh = lane / 32) dequantises chunk 2g + hh of weight row j for
// group g: its 4 words are the B operands of the 4 MFMAs of the group, the K
// order inside a group permuted the same way for A, which reads 16 bytes of
// activation row j at column 64g + 32hh + 8q for MFMA q.  Items are taken in
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

// 8 int4 weights (one word of two's-complement nibbles, element 2b in the low
// nibble of byte b) times their group scale s, each product exact in fp32
// ((n - 8) * s with n = q + 8), rounded to bf16.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s, float m8s) {
  uint32_t x = w ^ 0x88888888u;
  uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
  asm("" : "+v"(lo), "+v"(hi));  // byte conversions stay single instructions
  bf16x8 r;
  r[0] = (__bf16)__builtin_fmaf((float)(lo & 0xFFu), s, m8s);
  r[1] = (__bf16)__builtin_fmaf((float)(hi & 0xFFu), s, m8s);
  r[2] = (__bf16)__builtin_fmaf((float)((lo >> 8) & 0xFFu), s, m8s);
  r[3] = (__bf16)__builtin_fmaf((float)((hi >> 8) & 0xFFu), s, m8s);
  r[4] = (__bf16)__builtin_fmaf((float)((lo >> 16) & 0xFFu), s, m8s);
  r[5] = (__bf16)__builtin_fmaf((float)((hi >> 16) & 0xFFu), s, m8s);
  r[6] = (__bf16)__builtin_fmaf((float)(lo >> 24), s, m8s);
  r[7] = (__bf16)__builtin_fmaf((float)(hi >> 24), s, m8s);
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &v) { return __builtin_bit_cast(bf16x8, v); }

// ------------------------------------------------------------- M-block list
// One wave: for each slot (unique routed expert in union order, then the
// shared expert) its rows split into M-blocks of kMB; entries (expert, first
// row, rows).  Rows of routed slots are pair positions, those of the shared
// expert are T*k + token.
__global__ __launch_bounds__(64) void k_mblocks(Dims D, UnionDev U, int4 *__restrict__ list,
                                                int32_t *__restrict__ count, int max_entries) {
  const int lane = threadIdx.x;
  const int nu = clamp_nu(U.n_unique, D);
  const int slots = nu + (D.n_shared > 0 ? 1 : 0);
  int running = 0;
  for (int base = 0; base < slots; base += 64) {
    const int s = base + lane;
    int e = 0, p0 = 0, p1 = 0, cnt = 0, row0 = 0;
    if (s < slots && resolve_slot(D, U, nu, s, e, p0, p1)) {
      row0 = s < nu ? p0 : D.T * D.k;
      cnt = (p1 - p0 + kMB - 1) / kMB;
    }
    int inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    const int pos = running + inc - cnt;
    for (int b = 0; b < cnt; ++b)
      if (pos + b < max_entries) list[pos + b] = make_int4(e, row0 + b * kMB, min(kMB, p1 - p0 - b * kMB), 0);
    running += __shfl(inc, 63, 64);
  }
  if (lane == 0) *count = running < max_entries ? running : max_entries;
}

// ------------------------------------------------------- activation gather
// Row r of xb = bf16(x[token of row r]): rows [0, T*k) follow the pair order of
// the union lists, rows T*k + t hold token t for the shared expert.
__global__ __launch_bounds__(256) void k_gather_bf16(const float *__restrict__ x, Dims D, UnionDev U,
                                                     uint16_t *__restrict__ xb) {
  const int tk = D.T * D.k;
  const int rows = tk + (D.n_shared > 0 ? D.T : 0);
  for (int row = blockIdx.x; row < rows; row += gridDim.x) {
    int t = row < tk ? U.pair_token[row] : row - tk;
    const bool ok = t >= 0 && t < D.T;
    if (!ok) t = 0;
    const float *src = x + (size_t)t * D.d;
    uint16_t *dst = xb + (size_t)row * D.d;
    for (int c = 8 * threadIdx.x; c < D.d; c += 8 * 256) {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      if (ok) {
        a = *(const float4 *)(src + c);
        b = *(const float4 *)(src + c + 4);
      }
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
template <bool GATEUP>
__global__ __launch_bounds__(256) void k_gemm_mfma(LayerDev L, Dims D, const uint16_t *__restrict__ A,
                                                   const int4 *__restrict__ list, const int32_t *__restrict__ count,
                                                   int max_entries, uint16_t *__restrict__ hb,
                                                   float *__restrict__ y) {
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
  for (int base = 0; base < items; base += gridDim.x) {
    const int item = base + slot_in_round;
    if (item >= items) continue;
    const int mb = item / ntiles, nt = item - mb * ntiles;
    const int4 ent = list[mb];
    const int e = ent.x, row0 = ent.y, rc = ent.z;
    if (32 * wave + nt * kNT >= nrows) continue;  // whole wave past the last weight row
    const int gr = nt * kNT + 32 * wave + j;        // weight row of this lane
    const int tile = gr >> 3, r = gr & 7;
    const uint8_t *base_e = L.experts + (size_t)e * L.expert_stride;
    const uint8_t *nib = base_e + (GATEUP ? EL.gu_nib : EL.dn_nib);
    const uint16_t *sc = (const uint16_t *)(base_e + (GATEUP ? EL.gu_sc : EL.dn_sc)) + (size_t)tile * G * 8 + r;
    const int nmt = (rc + 31) >> 5;  // M-tiles holding rows (1..4)
    const uint16_t *arow[4];
    bool aok[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int rr = 32 * mt + j;
      aok[mt] = rr < rc;
      arow[mt] = A + (size_t)(row0 + (aok[mt] ? rr : 0)) * K + 32 * hh;
    }
    f32x16 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt][v] = 0.0f;

    uint4 Wn = *(const uint4 *)(nib + chunk_offset(tile, K, hh, r));
    float sn = (float)__builtin_bit_cast(_Float16, sc[0]);
    for (int g = 0; g < G; ++g) {
      const uint4 W = Wn;
      const float s = sn;
      if (g + 1 < G) {
        Wn = *(const uint4 *)(nib + chunk_offset(tile, K, 2 * (g + 1) + hh, r));
        sn = (float)__builtin_bit_cast(_Float16, sc[(size_t)(g + 1) * 8]);
      }
      const float m8s = -8.0f * s;
      const bf16x8 b0 = dequant8(W.x, s, m8s), b1 = dequant8(W.y, s, m8s);
      const bf16x8 b2 = dequant8(W.z, s, m8s), b3 = dequant8(W.w, s, m8s);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt < nmt) {
          uint4 a[4];
          const uint4 *ap = (const uint4 *)(arow[mt] + 64 * g);
#pragma unroll
          for (int q = 0; q < 4; ++q) a[q] = aok[mt] ? ap[q] : make_uint4(0u, 0u, 0u, 0u);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[0]), b0, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[1]), b1, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[2]), b2, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[3]), b3, acc[mt], 0, 0, 0);
        }
      }
    }

    // Epilogue.  Accumulator element v of lane (j, hh) is row 8(v/4) + 4hh + v%4
    // of the M-tile, column j (weight row gr).
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt < nmt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rr = 32 * mt + 8 * (v >> 2) + 4 * hh + (v & 3);
          const float val = acc[mt][v];
          if (GATEUP) {
            // tile rows 0-3 are gate rows, 4-7 the up rows of the same features
            const float up = __shfl_down(val, 4, 64);
            if ((j & 7) < 4 && rr < rc) {
              const int feat = 4 * tile + (j & 3);
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

// ---------------------------------------------------------------- launchers

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

hipError_t launch_gather_bf16(const float *x, const Dims &D, const UnionDev &U, uint16_t *xb, hipStream_t s) {
  const int rows = D.T * D.k + (D.n_shared > 0 ? D.T : 0);
  if (rows <= 0) return hipSuccess;
  k_gather_bf16<<<rows < 8192 ? rows : 8192, 256, 0, s>>>(x, D, U, xb);
  return hipGetLastError();
}

// Blocks of the persistent grid: a multiple of 8 (one share per XCD).
static int mfma_grid(int max_entries, int ntiles) {
  const long items = (long)max_entries * ntiles;
  long g = 1024;
  if (items < g) g = (items + 7) / 8 * 8;
  return (int)(g < 8 ? 8 : g);
}

hipError_t launch_gateup_mfma(const LayerDev &L, const Dims &D, const uint16_t *xb, const int4 *list,
                              const int32_t *count, int max_entries, uint16_t *hb, hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  const int ntiles = (2 * D.f + kNT - 1) / kNT;
  k_gemm_mfma<true><<<mfma_grid(max_entries, ntiles), 256, 0, s>>>(L, D, xb, list, count, max_entries, hb, nullptr);
  return hipGetLastError();
}

hipError_t launch_down_mfma(const LayerDev &L, const Dims &D, const uint16_t *hb, const int4 *list,
                            const int32_t *count, int max_entries, float *y, hipStream_t s) {
  if (D.T <= 0) return hipSuccess;
  const int ntiles = (D.d + kNT - 1) / kNT;
  k_gemm_mfma<false><<<mfma_grid(max_entries, ntiles), 256, 0, s>>>(L, D, hb, list, count, max_entries, nullptr, y);
  return hipGetLastError();
}

}  // namespace colimoe
