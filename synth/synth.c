/*
 * synth.c - seeded, counter-based synthetic inputs for the int4 routed-expert
 * MoE layer (test and benchmark fixture; not part of the compute path).
 *
 * Every value is a pure function of (seed, stream, counter), so any expert of
 * any layer can be regenerated on its own and the host never has to hold a
 * whole multi-layer model.  The mixing function is SplitMix64 (Steele, Lea and
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014).
 *
 * This file holds no arithmetic of the MoE method itself: it only draws
 * numbers and writes them in the canonical container format that the
 * library's loader and the CPU oracle each decode on their own.
 *
 * Canonical expert blob (one routed or shared expert, d = hidden size,
 * f = intermediate size, group size 64 along each row's input dimension):
 *   [gate nibbles  f*d/2 B][gate scales f*(d/64) fp16]
 *   [up   nibbles  f*d/2 B][up   scales f*(d/64) fp16]
 *   [down nibbles  d*f/2 B][down scales d*(f/64) fp16]
 * Matrices are row-major with rows = outputs (gate/up: [f][d], down: [d][f]).
 * Byte i of a row holds element 2i in bits 0-3 and element 2i+1 in bits 4-7,
 * each a 4-bit two's-complement integer in [-8, 7].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of one stream: (seed, stream id). */
uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GOLDEN) ^ (stream * GOLDEN + 0xD1B54A32D192ED03ULL));
}

/* Element `i` of stream `key`: the SplitMix64 output at state key + (i+1)*gamma. */
uint64_t synth_u64(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

/* Uniform double in (0, 1] from the top 53 bits. */
static inline double u01(uint64_t h) { return ((double)(h >> 11) + 1.0) * (1.0 / 9007199254740992.0); }

/* Stream ids.  expert == E denotes the always-on shared expert. */
enum { T_GATE_NIB = 0, T_GATE_SC, T_UP_NIB, T_UP_SC, T_DOWN_NIB, T_DOWN_SC, T_ROUTER = 8, T_ZIPF = 9, T_ACT = 10 };
uint64_t synth_stream(int layer, int expert, int tensor) {
  return (((uint64_t)(uint32_t)layer << 24) | ((uint64_t)(uint32_t)expert << 4) | (uint64_t)tensor) + 1;
}

/* Standard normal, element i of a stream (Box-Muller on two counter draws). */
static inline double normal_at(uint64_t key, uint64_t i) {
  double u1 = u01(synth_u64(key, 2 * i)), u2 = u01(synth_u64(key, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

/* Round a positive normal-range double to IEEE binary16 bits, ties to even.
 * Only used for the scales, which lie in [0.005, 0.02]. */
static uint16_t encode_half_pos_normal(double v) {
  int e;
  double m = frexp(v, &e); /* v = m * 2^e, m in [0.5, 1) */
  double frac = (m * 2.0 - 1.0) * 1024.0; /* 10-bit fraction, exact scaling */
  double r = nearbyint(frac);             /* default rounding mode: ties to even */
  uint32_t bits = ((uint32_t)(e - 1 + 15) << 10) + (uint32_t)r; /* carry bumps the exponent */
  return (uint16_t)bits;
}

size_t synth_expert_bytes(int d, int f) {
  size_t w = (size_t)d * (size_t)f;
  return 3 * (w / 2 + (w / 64) * 2);
}

static void fill_nibbles(uint64_t key, uint8_t *dst, size_t nbytes) {
  size_t nw = nbytes / 8;
  for (size_t i = 0; i < nw; ++i) {
    uint64_t h = synth_u64(key, i);
    memcpy(dst + 8 * i, &h, 8); /* little-endian host */
  }
  if (nbytes % 8) {
    uint64_t h = synth_u64(key, nw);
    memcpy(dst + 8 * nw, &h, nbytes % 8);
  }
}

static void fill_scales(uint64_t key, uint8_t *dst, size_t n, double lo, double hi) {
  for (size_t i = 0; i < n; ++i) {
    double u = (double)(synth_u64(key, i) >> 11) * (1.0 / 9007199254740992.0); /* [0,1) */
    uint16_t h = encode_half_pos_normal(lo + (hi - lo) * u);
    memcpy(dst + 2 * i, &h, 2);
  }
}

/* One canonical expert blob (layout above), int4 uniform over [-8, 7],
 * scales U(lo, hi) rounded to fp16. */
void synth_expert_blob(uint64_t seed, int layer, int expert, int d, int f, double sc_lo, double sc_hi,
                       uint8_t *blob) {
  size_t w = (size_t)d * (size_t)f, nb = w / 2, ns = w / 64;
  uint8_t *p = blob;
  static const int tnib[3] = {T_GATE_NIB, T_UP_NIB, T_DOWN_NIB};
  static const int tsc[3] = {T_GATE_SC, T_UP_SC, T_DOWN_SC};
  for (int m = 0; m < 3; ++m) {
    fill_nibbles(synth_key(seed, synth_stream(layer, expert, tnib[m])), p, nb);
    p += nb;
    fill_scales(synth_key(seed, synth_stream(layer, expert, tsc[m])), p, ns, sc_lo, sc_hi);
    p += ns * 2;
  }
}

/* int8 container: the same blob layout with one byte per weight, uniform
 * over [-128, 127] (the hash bytes read as two's complement), scales
 * U(lo, hi) rounded to fp16. */
size_t synth_expert_bytes_i8(int d, int f) {
  size_t w = (size_t)d * (size_t)f;
  return 3 * (w + (w / 64) * 2);
}

void synth_expert_blob_i8(uint64_t seed, int layer, int expert, int d, int f, double sc_lo, double sc_hi,
                          uint8_t *blob) {
  size_t w = (size_t)d * (size_t)f, ns = w / 64;
  uint8_t *p = blob;
  static const int tq[3] = {T_GATE_NIB, T_UP_NIB, T_DOWN_NIB};
  static const int tsc[3] = {T_GATE_SC, T_UP_SC, T_DOWN_SC};
  for (int m = 0; m < 3; ++m) {
    fill_nibbles(synth_key(seed ^ 0x1808ULL, synth_stream(layer, expert, tq[m])), p, w);
    p += w;
    fill_scales(synth_key(seed ^ 0x1808ULL, synth_stream(layer, expert, tsc[m])), p, ns, sc_lo, sc_hi);
    p += ns * 2;
  }
}

void synth_expert_blobs_i8(uint64_t seed, int layer, int e0, int e1, int d, int f, double sc_lo, double sc_hi,
                           uint8_t *out) {
  size_t be = synth_expert_bytes_i8(d, f);
#pragma omp parallel for schedule(dynamic, 1)
  for (int e = e0; e < e1; ++e) synth_expert_blob_i8(seed, layer, e, d, f, sc_lo, sc_hi, out + (size_t)(e - e0) * be);
}

/* Experts [e0, e1) of one layer into consecutive blobs; OpenMP over experts. */
void synth_expert_blobs(uint64_t seed, int layer, int e0, int e1, int d, int f, double sc_lo, double sc_hi,
                        uint8_t *out) {
  size_t be = synth_expert_bytes(d, f);
#pragma omp parallel for schedule(dynamic, 1)
  for (int e = e0; e < e1; ++e) synth_expert_blob(seed, layer, e, d, f, sc_lo, sc_hi, out + (size_t)(e - e0) * be);
}

/* Router matrix [E][d] fp32, entries std * N(0,1). */
void synth_router(uint64_t seed, int layer, int E, int d, double std, float *out) {
  uint64_t key = synth_key(seed, synth_stream(layer, 0, T_ROUTER));
  size_t n = (size_t)E * (size_t)d;
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < (long long)n; ++i) out[i] = (float)(std * normal_at(key, (uint64_t)i));
}

typedef struct { uint64_t h; int e; } hk_t;
static int hk_cmp(const void *a, const void *b) {
  const hk_t *x = (const hk_t *)a, *y = (const hk_t *)b;
  if (x->h != y->h) return x->h < y->h ? -1 : 1;
  return x->e - y->e;
}

/* Zipf(s) prior over experts as an additive logit bias: a seeded permutation
 * pi of the experts, b_e = -s * ln(pi(e) + 1). */
void synth_zipf_bias(uint64_t seed, int layer, int E, double s, float *out) {
  uint64_t key = synth_key(seed, synth_stream(layer, 0, T_ZIPF));
  hk_t *v = (hk_t *)malloc(sizeof(hk_t) * (size_t)E);
  for (int e = 0; e < E; ++e) { v[e].h = synth_u64(key, (uint64_t)e); v[e].e = e; }
  qsort(v, (size_t)E, sizeof(hk_t), hk_cmp);
  for (int r = 0; r < E; ++r) out[v[r].e] = (float)(-s * log((double)r + 1.0));
  free(v);
}

/* Activations [T][d] fp32: x_t = sqrt(rho) z_0 + sqrt(1-rho) z_t with z iid N(0,1)
 * (rho = 0 gives iid rows).  `stream` separates independent draws. */
void synth_activations(uint64_t seed, int stream, int T, int d, double rho, float *out) {
  uint64_t kc = synth_key(seed, synth_stream(stream, 0xFFFF, T_ACT));
  uint64_t kt = synth_key(seed, synth_stream(stream, 0, T_ACT));
  double a = sqrt(rho), b = sqrt(1.0 - rho);
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < (long long)T * d; ++i) {
    double z = normal_at(kt, (uint64_t)i);
    if (rho != 0.0) z = a * normal_at(kc, (uint64_t)(i % d)) + b * z;
    out[i] = (float)z;
  }
}
