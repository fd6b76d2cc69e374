/*
 * oracle.c - plain, slow CPU reference of the int4 routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  It shares no code,
 * header, table or constant with the HIP library and includes none of it.
 *
 * Sources (cited by page title and section):
 *   [A] "Colibrì: running a 744B MoE model on a laptop with 2400 lines of pure C"
 *       (kechuai.cn article)
 *   [P] "colibrì" project profile (gh.puless.com)
 *   [D] "colibrì: 1300 lines of C, a 25 GB laptop, a 744-billion-parameter model"
 *       (SSP GitHub Daily #091, jsqmd.com)
 *
 * What the pages fix: a router picks 8 of 256 experts per layer ([A] §1; [D] §3);
 * each expert is three adjacent matrices ([A] §2); the container is int4 with
 * group size 64 ([P] "aggressive optimisation, conservative correctness");
 * at batch 1 the weights are dequantised and multiplied in floating point
 * ([D] §4, highlight 4); the shared expert is used for every token ([D] §3);
 * batched positions read each unique expert once ([A] §2); precision and
 * routing are never changed silently ([A] §4).  Where the pages are silent
 * (nibble order, signedness, matrix orientation, gating function, tie order,
 * activation) the plainest reading is taken; each one is named at the function
 * that depends on it.
 *
 * Everything here is the definition written out in fp64: sums run
 * sequentially over the input index, exp() is libm's.  OpenMP splits only
 * independent output rows, so results do not depend on the thread count.
 *
 * Parity pins: every function below is pinned by tests that do not call it
 * to check itself (exhaustive decode tables, closed forms, library sorts,
 * dense special cases, brute force, exact sums).  The end-to-end values at
 * the full-size workloads are pinned only through those parts: the pages
 * print no worked numeric example of the layer.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GS 64 /* elements per scale group ([P] "conservative correctness": gs64) */

/* Container width: 4 (int4, the default) or 8 (int8 gs64: the pages keep the
 * MTP head in int8 because int4 lost too much precision there, [P] lessons
 * on record and [D] §4 highlight 2; here offered for expert weights).  Reading of the int8 container: the same blob layout
 * with one two's-complement byte per weight, row-major, and the same fp16
 * group scales. */
static int g_bits = 4;
void oracle_set_bits(int bits) { g_bits = bits == 8 ? 8 : 4; }

/* ---------------------------------------------------------------- decoding */

/* O1: one int4 element.  Reading: byte i of a row holds element 2i in its low
 * four bits and element 2i+1 in its high four bits; each is a 4-bit two's
 * complement integer in [-8, 7] with no zero-point. */
int oracle_nibble(uint8_t byte, int high) {
  int n = high ? (byte >> 4) & 15 : byte & 15;
  return n >= 8 ? n - 16 : n;
}

/* O2: IEEE 754 binary16 -> double, exactly (normals, subnormals, zeros,
 * infinities, NaN), from the format's definition. */
double oracle_half(uint16_t h) {
  int sign = (h >> 15) & 1, ex = (h >> 10) & 31, man = h & 1023;
  double v;
  if (ex == 31)
    v = man ? NAN : INFINITY;
  else if (ex == 0)
    v = ldexp((double)man, -24); /* subnormal: man * 2^-14 * 2^-10 */
  else
    v = ldexp((double)(1024 + man), ex - 25); /* (1 + man/1024) * 2^(ex-15) */
  return sign ? -v : v;
}

static inline uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* O3: dequantised element W[r][c] = q[r][c] * s[r][c/64] of a row-major
 * [rows][cols] matrix (groups run along each row's input dimension). */
double oracle_weight(const uint8_t *nib, const uint8_t *sc, int rows, int cols, int r, int c) {
  (void)rows;
  int q;
  if (g_bits == 8) {
    const uint8_t b = nib[(size_t)r * (size_t)cols + (size_t)c];
    q = b >= 128 ? (int)b - 256 : (int)b; /* two's complement byte */
  } else {
    size_t rowb = (size_t)cols / 2;
    uint8_t b = nib[(size_t)r * rowb + (size_t)(c / 2)];
    q = oracle_nibble(b, c & 1);
  }
  int g = c / GS;
  double s = oracle_half(rd16(sc + 2 * ((size_t)r * (size_t)(cols / GS) + (size_t)g)));
  return (double)q * s;
}

/* Whole matrix, dequantised into W[rows][cols]. */
void oracle_dequant(const uint8_t *nib, const uint8_t *sc, int rows, int cols, double *W) {
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c) W[(size_t)r * cols + c] = oracle_weight(nib, sc, rows, cols, r, c);
}

/* y = W x, and optionally yabs[r] = sum_c |W[r][c] x[c]|.  Sequential in c. */
void oracle_matvec(const uint8_t *nib, const uint8_t *sc, int rows, int cols, const double *x, double *y,
                   double *yabs) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    double acc = 0.0, aab = 0.0;
    for (int c = 0; c < cols; ++c) {
      double p = oracle_weight(nib, sc, rows, cols, r, c) * x[c];
      acc += p;
      aab += fabs(p);
    }
    y[r] = acc;
    if (yabs) yabs[r] = aab;
  }
}

/* Canonical blob sections ([A] §2: an expert's three matrices sit side by
 * side).  Reading: gate, up, down in that order, each followed by its fp16
 * scales; gate/up are [f][d], down is [d][f], rows being outputs. */
typedef struct {
  const uint8_t *gn, *gs, *un, *us, *dn, *ds;
} blob_view;

static blob_view view_blob(const uint8_t *blob, int d, int f) {
  size_t w = (size_t)d * (size_t)f, nb = g_bits == 8 ? w : w / 2, ns = (w / GS) * 2;
  blob_view v;
  v.gn = blob;
  v.gs = v.gn + nb;
  v.un = v.gs + ns;
  v.us = v.un + nb;
  v.dn = v.us + ns;
  v.ds = v.dn + nb;
  return v;
}

size_t oracle_expert_bytes(int d, int f) {
  size_t w = (size_t)d * (size_t)f;
  return 3 * ((g_bits == 8 ? w : w / 2) + (w / GS) * 2);
}

/* --------------------------------------------------------------- the layer */

/* SiLU(z) = z * sigmoid(z) = z / (1 + e^-z). */
double oracle_silu(double z) {
  return z / (1.0 + exp(-z));
}

/* O7: one expert's feed-forward.  g = Wg x, u = Wu x, h = SiLU(g) * u,
 * y = Wd h (reading: SwiGLU, the pages name no activation).  Any output
 * pointer may be NULL except y; yabs receives sum_c |Wd[r][c] h[c]|. */
void oracle_expert(const uint8_t *blob, int d, int f, const double *x, double *g, double *u, double *h,
                   double *y, double *yabs) {
  blob_view v = view_blob(blob, d, f);
  double *gg = (double *)malloc(sizeof(double) * (size_t)f);
  double *uu = (double *)malloc(sizeof(double) * (size_t)f);
  double *hh = (double *)malloc(sizeof(double) * (size_t)f);
  oracle_matvec(v.gn, v.gs, f, d, x, gg, NULL);
  oracle_matvec(v.un, v.us, f, d, x, uu, NULL);
  for (int i = 0; i < f; ++i) hh[i] = oracle_silu(gg[i]) * uu[i];
  oracle_matvec(v.dn, v.ds, d, f, hh, y, yabs);
  if (g) memcpy(g, gg, sizeof(double) * (size_t)f);
  if (u) memcpy(u, uu, sizeof(double) * (size_t)f);
  if (h) memcpy(h, hh, sizeof(double) * (size_t)f);
  free(gg);
  free(uu);
  free(hh);
}

/* O4: router logits l[e] = sum_c R[e][c] x[c] + b[e] in fp64 (for fp32 x the
 * products are exact).  8 of 256 experts are then chosen ([A] §1). */
void oracle_router(const float *R, const float *bias, const double *x, int E, int d, double *l) {
#pragma omp parallel for schedule(static)
  for (int e = 0; e < E; ++e) {
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += (double)R[(size_t)e * d + c] * x[c];
    if (bias) acc += (double)bias[e];
    l[e] = acc;
  }
}

/* Order used for selection: larger logit first; an exact tie goes to the
 * lower expert index (reading: deterministic routing, [A] §4). */
static const double *g_sort_l;
static int before(int a, int b, const double *l) {
  if (l[a] != l[b]) return l[a] > l[b];
  return a < b;
}
static int cmp_sort(const void *pa, const void *pb) {
  int a = *(const int *)pa, b = *(const int *)pb;
  if (before(a, b, g_sort_l)) return -1;
  if (before(b, a, g_sort_l)) return 1;
  return 0;
}

/* O5a: top-k by a full sort of all experts. */
void oracle_topk_sort(const double *l, int E, int k, int32_t *idx) {
  int *ord = (int *)malloc(sizeof(int) * (size_t)E);
  for (int e = 0; e < E; ++e) ord[e] = e;
  g_sort_l = l;
  qsort(ord, (size_t)E, sizeof(int), cmp_sort);
  for (int j = 0; j < k; ++j) idx[j] = ord[j];
  free(ord);
}

/* O5b: top-k by k passes of "best remaining" (independent of the sort). */
void oracle_topk_select(const double *l, int E, int k, int32_t *idx) {
  char *taken = (char *)calloc((size_t)E, 1);
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e)
      if (!taken[e] && (best < 0 || before(e, best, l))) best = e;
    idx[j] = best;
    taken[best] = 1;
  }
  free(taken);
}

/* Gate weights: softmax over the k selected logits only (reading: no
 * renormalisation or scaling beyond that).  w_j = e^(l_j - m) / sum_i e^(l_i - m). */
void oracle_softmax_selected(const double *l, int E, const int32_t *idx, int k, double *w) {
  double m = -INFINITY, s = 0.0;
  (void)E;
  for (int j = 0; j < k; ++j) m = fmax(m, l[idx[j]]);
  for (int j = 0; j < k; ++j) s += exp(l[idx[j]] - m);
  for (int j = 0; j < k; ++j) w[j] = exp(l[idx[j]] - m) / s;
}

/* Adaptive expert top-p ([D] key tuning parameters: "topp=0.7", an adaptive
 * expert top-p that reads 30-40% fewer experts; [D] §4: top-p changes which
 * experts are read).  Reading: take the k experts in top-k order with their
 * gate weights w (softmax over the k selected), keep the shortest prefix
 * whose weight sum reaches p (at least the first expert), and give the kept
 * experts the softmax over their own logits.  Dropped entries become idx -1,
 * w 0.  p >= 1 keeps all k.  Returns the number kept. */
int oracle_expert_top_p(const double *l, int E, int k, double p, int32_t *idx, double *w) {
  int m = k;
  if (p < 1.0) {
    double cum = 0.0;
    m = 0;
    while (m < k && (m == 0 || cum < p)) {
      cum += w[m];
      ++m;
    }
  }
  oracle_softmax_selected(l, E, idx, m, w);
  for (int j = m; j < k; ++j) {
    idx[j] = -1;
    w[j] = 0.0;
  }
  return m;
}

/* O6: batch-union ([A] §2: batched positions read each unique expert once).
 * ids: distinct experts, ascending; offsets[u]..offsets[u+1]: that expert's
 * (token, slot) pairs, ordered by token; pair_of[t*k + j]: position of the
 * pair (t, j), -1 for a slot dropped by expert top-p (idx -1).  Returns the
 * number of distinct experts. */
int oracle_union(const int32_t *idx, int T, int k, int E, int32_t *ids, int32_t *offsets, int32_t *pair_token,
                 int32_t *pair_slot, int32_t *pair_of) {
  int n = 0, p = 0;
  offsets[0] = 0;
  for (size_t i = 0; i < (size_t)T * k; ++i) pair_of[i] = -1;
  for (int e = 0; e < E; ++e) {
    int cnt = 0;
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j)
        if (idx[(size_t)t * k + j] == e) {
          pair_token[p] = t;
          pair_slot[p] = j;
          pair_of[(size_t)t * k + j] = p;
          ++p;
          ++cnt;
        }
    if (cnt) {
      ids[n] = e;
      offsets[n + 1] = p;
      ++n;
    }
  }
  return n;
}

/* RMSNorm with unit weight: x = r / sqrt(mean(r^2) + eps). */
void oracle_rmsnorm(const double *r, int d, double eps, double *x) {
  double ss = 0.0;
  for (int c = 0; c < d; ++c) ss += r[c] * r[c];
  double inv = 1.0 / sqrt(ss / (double)d + eps);
  for (int c = 0; c < d; ++c) x[c] = r[c] * inv;
}

/* O8: one token through one MoE layer.
 *   x        [d]   fp64 activations the router and the experts see
 *   experts  E pointers to canonical blobs (only selected ones are read)
 *   shared   blob of the always-on shared expert or NULL ([D] §3)
 *   idx, w   the routing to apply (k entries; idx -1 is a dropped slot)
 *   residual [d]   the stream the combine adds into
 * out = residual + sum_j w_j y_j + y_shared, and
 * l1[r] = |residual_r| + sum_j |w_j| sum_c |Wd_j[r][c] h_j[c]| + sum_c |Wd_sh[r][c] h_sh[c]|
 * (the per-output L1 norm of the products, the scale of the bf16 bound). */
int oracle_moe_token(const double *x, int d, int f, int k, const uint8_t *const *experts, const uint8_t *shared,
                     const int32_t *idx, const double *w, const double *residual, double *out, double *l1) {
  double *y = (double *)malloc(sizeof(double) * (size_t)d);
  double *ya = (double *)malloc(sizeof(double) * (size_t)d);
  for (int r = 0; r < d; ++r) {
    out[r] = residual[r];
    if (l1) l1[r] = fabs(residual[r]);
  }
  for (int j = 0; j < k; ++j) {
    if (idx[j] < 0) continue; /* dropped by expert top-p: contributes nothing */
    const uint8_t *b = experts[idx[j]];
    if (!b) {
      free(y);
      free(ya);
      return -1; /* caller did not supply a selected expert */
    }
    oracle_expert(b, d, f, x, NULL, NULL, NULL, y, ya);
    for (int r = 0; r < d; ++r) {
      out[r] += w[j] * y[r];
      if (l1) l1[r] += fabs(w[j]) * ya[r];
    }
  }
  if (shared) {
    oracle_expert(shared, d, f, x, NULL, NULL, NULL, y, ya);
    for (int r = 0; r < d; ++r) {
      out[r] += y[r];
      if (l1) l1[r] += ya[r];
    }
  }
  free(y);
  free(ya);
  return 0;
}

/* Route one token: logits, top-k by sort (cross-checked against selection),
 * softmax over the selected.  Returns -2 if the two top-k methods disagree. */
int oracle_route_token(const float *R, const float *bias, const double *x, int E, int d, int k, double *logits,
                       int32_t *idx, double *w) {
  int32_t *alt = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
  oracle_router(R, bias, x, E, d, logits);
  oracle_topk_sort(logits, E, k, idx);
  oracle_topk_select(logits, E, k, alt);
  int rc = memcmp(alt, idx, sizeof(int32_t) * (size_t)k) ? -2 : 0;
  free(alt);
  oracle_softmax_selected(logits, E, idx, k, w);
  return rc;
}
