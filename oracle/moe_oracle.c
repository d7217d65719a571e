/* CPU ORACLE for one GLM-5.2-style (glm_moe_dsa) MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, fp64 definition of what
 * the layer computes.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the GPU library never does, and the two share
 * no code (this file has its own types, decoders and loops).
 *
 * Sources (web pages; cited by title and section):
 *  [PORT]   "GLM-5.2 on a 32 GB Mac - native MLX port of the Colibri hierarchy"
 *           (mlx-bun design doc): section "N1. GLM-5.2 graph" (the biased sigmoid
 *           scores choose the experts and the unbiased ones weigh them, an exact
 *           top-8, an optional renormalisation, the routed scale, and a shared
 *           expert computed beside the routed ones);
 *           "G2 implementation status" (equal keys go to the lower expert index;
 *           the expert weights come from the sigmoid without its bias; the routed
 *           sum is scaled; the shared expert enters with weight one; an int4
 *           nibble n stands for n - 8; weights are dequantised and then
 *           multiplied and accumulated in f32).
 *  [README] colibri README, "What's implemented" (the sigmoid noaux_tc router of
 *           the DeepSeek-V3 kind with its scaling factor, and the shared expert).
 *  [MODELS] "Model support" doc, section 4.3 UniversalMoE (top-k, norm_topk_probs,
 *           sigmoid scoring, routing scale, shared expert, grouped routing in the
 *           deepseek_v3 style) and section 6.4 GLM-5.2.
 *
 * Readings where the pages are silent (all of them listed in the design notes):
 *  R1 groups are n_group contiguous blocks of E/n_group experts; a group's score
 *     is the sum of its two largest selection keys; the topk_group best groups
 *     are kept (ties: lower group index) and experts outside them are excluded.
 *  R2 ranking compares fp32-rounded keys key_e = fp32(sigmoid(l_e) + bias_e) with
 *     the sigmoid and the sum in fp64; a group score is fp32(k1 + k2); exact ties
 *     go to the lower expert (group) index.  idx is emitted in rank order.
 *  R3 w_j = s_j / sum_m s_m * rsf when norm_topk_prob, else s_j * rsf; no epsilon.
 *  R4 SwiGLU expert: h = silu(Wg x) * (Wu x), y_e = Wd h, silu(z) = z/(1+e^-z);
 *     no biases, no clamp.  Shared expert has weight 1, added after the routed sum.
 *  R5 int4 scales are fp16, one per 32 consecutive elements along the contraction.
 *  R6 weight formats ([PORT] "G2 implementation status", "G3 implementation
 *     status", "G4"): fmt 0 = int4, fp16 scale per 32 elements (R5); fmt 1 = int4
 *     with one fp32 scale per row (the production container's whole-row group:
 *     the group size is the row length); fmt 2 = signed int8 (two's complement
 *     bytes) with one fp32 scale per row (the MTP layer's routed experts).  In
 *     every format W[r,c] = q[r,c] * scale, exact in fp64.
 *  R7 int8 activations ([PORT] "G2 implementation status": the IDOT=1 setting
 *     of Colibri, an approximate mode in which every activation row becomes
 *     int8 ahead of its dot products with the packed int4 weights; [README]
 *     "Integer-dot kernels"): a row v of length n (the layer input of a token, and each
 *     expert's hidden activation h after it is rounded to fp32) becomes
 *     d = fp32(amax / 127) with amax = max |v| (fp32), q_c = rint(fp32(v_c / d))
 *     (ties to even; q = 0 for an all-zero row), and the matmul uses q_c * d
 *     (exact in fp64) in place of v_c.
 *  R8 bf16 operands (the library's matrix-core path, its own choice and not the
 *     pages'): for an expert so marked, the gate/up contraction sees the token's
 *     input rounded to bf16 and every weight rounded to fp32 and then to bf16,
 *     and the down contraction sees h rounded to fp32 and then to bf16 and its
 *     weights rounded the same way; all roundings to nearest, ties to even; the
 *     arithmetic stays fp64.  Which experts are marked is the caller's input
 *     (the library marks those a batch sends to its matrix cores).
 *
 * Parity pins: tests/test_oracle_pins.py (brute force, closed forms, invariants)
 * and tests/test_oracle_diag.py (the decision margins and the near-midpoint flag
 * on hand-built keys).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- decoders */

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1F;
  int frac = h & 0x3FF;
  double v;
  if (ex == 0) {
    v = ldexp((double)frac, -24); /* subnormal: frac * 2^-14 * 2^-10 */
  } else if (ex == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp(1024.0 + (double)frac, ex - 25); /* (1 + frac/1024) * 2^(ex-15) */
  }
  return sign ? -v : v;
}

/* bfloat16 is the upper half of an fp32 word. */
double oracle_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* int4 element c of a row of offset-binary nibbles: value = nibble - 8
 * (element 2j in the low nibble of byte j, 2j+1 in the high nibble). */
static int q_of(const uint8_t *row, int c) {
  uint8_t b = row[c >> 1];
  int u = (c & 1) ? (b >> 4) : (b & 0x0F);
  return u - 8;
}

/* Dequantised weight matrix [R, K]: W[r,c] = q[r,c] * s[r, c/gsz]  (exact in fp64). */
void oracle_dequant(int R, int K, int gsz, const uint8_t *q, const uint16_t *s, double *out) {
  for (int r = 0; r < R; ++r)
    for (int c = 0; c < K; ++c)
      out[(size_t)r * K + c] =
          (double)q_of(q + (size_t)r * (K / 2), c) * oracle_f16_to_f64(s[(size_t)r * (K / gsz) + c / gsz]);
}

/* One weight W[r,c] of an R x K matrix in format fmt (R6); q is the matrix's
 * bytes (K/2 per row for int4, K for int8), s its scales (fp16 bits [R, K/gsz]
 * for fmt 0, fp32 [R] otherwise). */
static double w_at(int fmt, int K, int gsz, const uint8_t *q, const void *s, int r, int c) {
  if (fmt == 0)
    return (double)q_of(q + (size_t)r * (K / 2), c) * oracle_f16_to_f64(((const uint16_t *)s)[(size_t)r * (K / gsz) + c / gsz]);
  double scale = (double)((const float *)s)[r];
  if (fmt == 1) return (double)q_of(q + (size_t)r * (K / 2), c) * scale;
  return (double)(int8_t)q[(size_t)r * K + c] * scale;
}

/* Dequantised [R, K] matrix in any format. */
void oracle_dequant_fmt(int fmt, int R, int K, int gsz, const uint8_t *q, const void *s, double *out) {
  for (int r = 0; r < R; ++r)
    for (int c = 0; c < K; ++c) out[(size_t)r * K + c] = w_at(fmt, K, gsz, q, s, r, c);
}

/* ------------------------------------------------------------------ router */

/* distance-from-midpoint test: is fp64 v within 2^-40 |v| of a point where
 * rounding to fp32 changes direction? */
static int near_f32_midpoint(double v) {
  float f = (float)v;
  if ((double)f == v || !isfinite(v)) return 0;
  float g = nextafterf(f, v > (double)f ? INFINITY : -INFINITY);
  double mid = 0.5 * ((double)f + (double)g);
  return fabs(v - mid) <= ldexp(fabs(v), -40);
}

static double ulp32(float f) {
  float g = nextafterf(fabsf(f), INFINITY);
  return (double)g - (double)fabsf(f);
}

/* Decision diagnostics per token. */
typedef struct {
  double expert_margin; /* key(k-th pick) - best excluded candidate key, fp32 values */
  double group_margin;  /* score(Gk-th group) - best dropped group score */
  int32_t flags;        /* bit0: a fp32 rounding near a midpoint could change a decision */
  int32_t n_candidates; /* experts in the kept groups */
} oracle_diag;

/* One token's selection from its logits l[E] (fp64).
 * Steps follow [PORT] N1 / G2 status and [MODELS] 4.3 with readings R1-R3. */
int oracle_select(int E, int G, int Gk, int k, double rsf, int norm, const double *logits,
                  const float *bias, int32_t *idx, double *w, double *s_out, oracle_diag *diag) {
  if (E <= 0 || G <= 0 || E % G || Gk < 1 || Gk > G || k < 1 || k > Gk * (E / G)) return -1;
  const int per = E / G;
  double *s = malloc(sizeof(double) * E);
  double *key64 = malloc(sizeof(double) * E);
  float *key = malloc(sizeof(float) * E);
  float *gscore = malloc(sizeof(float) * G);
  double *gscore64 = malloc(sizeof(double) * G);
  char *gkeep = calloc(G, 1), *taken = calloc(E, 1), *cand = calloc(E, 1);
  int flags = 0;

  /* sigmoid scores (unbiased) and biased selection keys */
  for (int e = 0; e < E; ++e) {
    s[e] = 1.0 / (1.0 + exp(-logits[e]));
    key64[e] = s[e] + (double)bias[e];
    key[e] = (float)key64[e];
    if (s_out) s_out[e] = s[e];
  }
  /* group score = sum of the two largest keys in the group */
  for (int j = 0; j < G; ++j) {
    int b1 = -1, b2 = -1;
    for (int e = j * per; e < (j + 1) * per; ++e) {
      if (b1 < 0 || key[e] > key[b1]) { b2 = b1; b1 = e; }
      else if (b2 < 0 || key[e] > key[b2]) { b2 = e; }
    }
    double sum = (double)key[b1] + (b2 >= 0 ? (double)key[b2] : 0.0);
    gscore64[j] = sum;
    gscore[j] = (float)sum;
  }
  /* keep the topk_group best groups (ties: lower group index) */
  float last_kept = 0.0f;
  for (int it = 0; it < Gk; ++it) {
    int best = -1;
    for (int j = 0; j < G; ++j)
      if (!gkeep[j] && (best < 0 || gscore[j] > gscore[best])) best = j;
    gkeep[best] = 1;
    last_kept = gscore[best];
  }
  double gmargin = INFINITY;
  for (int j = 0; j < G; ++j)
    if (!gkeep[j]) {
      double m = (double)last_kept - (double)gscore[j];
      if (m < gmargin) gmargin = m;
      if (m <= 2.0 * ulp32(last_kept)) {
        /* a near-tied group decision: sensitive if any score or key feeding it sits near a midpoint */
        for (int jj = 0; jj < G; ++jj)
          if ((gkeep[jj] && gscore[jj] == last_kept) || jj == j) {
            if (near_f32_midpoint(gscore64[jj])) flags |= 1;
            for (int e = jj * per; e < (jj + 1) * per; ++e)
              if (near_f32_midpoint(key64[e])) flags |= 1;
          }
      }
    }
  int ncand = 0;
  for (int e = 0; e < E; ++e)
    if (gkeep[e / per]) { cand[e] = 1; ++ncand; }
  /* top-k over the kept experts (ties: lower expert index), emitted in rank order */
  for (int it = 0; it < k; ++it) {
    int best = -1;
    for (int e = 0; e < E; ++e)
      if (cand[e] && !taken[e] && (best < 0 || key[e] > key[best])) best = e;
    taken[best] = 1;
    idx[it] = best;
  }
  /* sensitivity of the expert decisions: adjacent ranks and the cut-off */
  double emargin = INFINITY;
  for (int e = 0; e < E; ++e)
    if (cand[e] && !taken[e]) {
      double m = (double)key[idx[k - 1]] - (double)key[e];
      if (m < emargin) emargin = m;
    }
  for (int it = 0; it < k; ++it) {
    float a = key[idx[it]];
    for (int e = 0; e < E; ++e) {
      if (!cand[e] || e == idx[it]) continue;
      int later = !taken[e];
      for (int jt = it + 1; jt < k; ++jt) later |= (idx[jt] == e);
      if (!later) continue;
      if ((double)a - (double)key[e] <= ulp32(a) &&
          (near_f32_midpoint(key64[idx[it]]) || near_f32_midpoint(key64[e])))
        flags |= 1;
    }
  }
  /* weights from the unbiased sigmoid, renormalised and scaled */
  double denom = 0.0;
  for (int it = 0; it < k; ++it) denom += s[idx[it]];
  for (int it = 0; it < k; ++it) w[it] = norm ? s[idx[it]] / denom * rsf : s[idx[it]] * rsf;

  if (diag) {
    diag->expert_margin = emargin;
    diag->group_margin = gmargin;
    diag->flags = flags;
    diag->n_candidates = ncand;
  }
  free(s); free(key64); free(key); free(gscore); free(gscore64);
  free(gkeep); free(taken); free(cand);
  return 0;
}

/* logit l[t,e] = sum_h x[t,h] W[e,h], fp64, h ascending. x is fp32, or bf16 bits. */
static double x_at(const void *x, int x_is_bf16, size_t i) {
  return x_is_bf16 ? oracle_bf16_to_f64(((const uint16_t *)x)[i]) : (double)((const float *)x)[i];
}

int oracle_route(int S, int H, int E, int G, int Gk, int k, double rsf, int norm, int x_is_bf16,
                 const void *x, const float *W, const float *bias, int32_t *idx, double *w,
                 double *logits_out, oracle_diag *diag) {
  if (S < 0 || H <= 0) return -1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int t = 0; t < S; ++t) {
    double *l = malloc(sizeof(double) * E);
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h) acc += x_at(x, x_is_bf16, (size_t)t * H + h) * (double)W[(size_t)e * H + h];
      l[e] = acc;
      if (logits_out) logits_out[(size_t)t * E + e] = acc;
    }
    if (oracle_select(E, G, Gk, k, rsf, norm, l, bias, idx + (size_t)t * k, w + (size_t)t * k, NULL,
                      diag ? diag + t : NULL))
      bad = 1;
    free(l);
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------ expert FFN */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* R8: f rounded to the nearest bf16 (8 significant bits), ties to even; NaN stays
 * NaN, and a value beyond the largest bf16 becomes an infinity. */
float oracle_bf16_round(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return f; /* inf, NaN */
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  u &= 0xFFFF0000u;
  memcpy(&f, &u, 4);
  return f;
}
static double bf16_of(double v) { return (double)oracle_bf16_round((float)v); }

/* R7: v[n] (fp32 values) -> q[n] (int8 values) and the row's scale d; out[c] =
 * q_c * d in fp64.  The decisions are taken in fp32 (IEEE division). */
float oracle_quant_row(int n, const float *v, int8_t *q, double *out) {
  float amax = 0.0f;
  for (int c = 0; c < n; ++c) amax = fmaxf(amax, fabsf(v[c]));
  float d = amax / 127.0f;
  for (int c = 0; c < n; ++c) {
    float r = d > 0.0f ? rintf(v[c] / d) : 0.0f;
    if (q) q[c] = (int8_t)r;
    if (out) out[c] = (double)r * (double)d;
  }
  return d;
}

/* y[H] = Wd (silu(Wg x) * (Wu x)) for one token, fp64.  Matrices in the
 * interchange layout of format fmt (R6): gate/up [I, H], down [H, I].
 * h_out (optional) receives the [I] hidden activation. */
/* bf16 (R8): x is already rounded by the caller; the weights and h are rounded here. */
static void expert_ffn_impl(int fmt, int act_int8, int bf16, int H, int I, int gsz, const uint8_t *qg,
                            const void *sg, const uint8_t *qu, const void *su, const uint8_t *qd, const void *sd,
                            const double *x, double *y, double *h_out) {
  double *h = malloc(sizeof(double) * I);
#pragma omp parallel for schedule(static)
  for (int r = 0; r < I; ++r) {
    double g = 0.0, u = 0.0;
    for (int c = 0; c < H; ++c) {
      double wg = w_at(fmt, H, gsz, qg, sg, r, c), wu = w_at(fmt, H, gsz, qu, su, r, c);
      if (bf16) {
        wg = bf16_of(wg);
        wu = bf16_of(wu);
      }
      g += wg * x[c];
      u += wu * x[c];
    }
    h[r] = silu(g) * u;
  }
  if (h_out) memcpy(h_out, h, sizeof(double) * I);
  if (bf16)
    for (int c = 0; c < I; ++c) h[c] = bf16_of(h[c]);
  if (act_int8) { /* R7: the down projection sees h rounded to fp32, then quantised */
    float *h32 = malloc(sizeof(float) * I);
    for (int c = 0; c < I; ++c) h32[c] = (float)h[c];
    oracle_quant_row(I, h32, NULL, h);
    free(h32);
  }
#pragma omp parallel for schedule(static)
  for (int r = 0; r < H; ++r) {
    double acc = 0.0;
    for (int c = 0; c < I; ++c) {
      const double wd = w_at(fmt, I, gsz, qd, sd, r, c);
      acc += (bf16 ? bf16_of(wd) : wd) * h[c];
    }
    y[r] = acc;
  }
  free(h);
}

/* x is the activation the gate/up matmuls see (already quantised in R7 mode). */
void oracle_expert_ffn_fmt(int fmt, int H, int I, int gsz, const uint8_t *qg, const void *sg, const uint8_t *qu,
                           const void *su, const uint8_t *qd, const void *sd, const double *x, double *y,
                           double *h_out) {
  expert_ffn_impl(fmt, 0, 0, H, I, gsz, qg, sg, qu, su, qd, sd, x, y, h_out);
}

/* R7 mode: x (fp32 values) is quantised here; h_out receives h before its quantisation. */
void oracle_expert_ffn_int8act(int fmt, int H, int I, int gsz, const uint8_t *qg, const void *sg, const uint8_t *qu,
                               const void *su, const uint8_t *qd, const void *sd, const float *x, double *y,
                               double *h_out) {
  double *xq = malloc(sizeof(double) * H);
  oracle_quant_row(H, x, NULL, xq);
  expert_ffn_impl(fmt, 1, 0, H, I, gsz, qg, sg, qu, su, qd, sd, xq, y, h_out);
  free(xq);
}

void oracle_expert_ffn(int H, int I, int gsz, const uint8_t *qg, const uint16_t *sg, const uint8_t *qu,
                       const uint16_t *su, const uint8_t *qd, const uint16_t *sd, const double *x, double *y,
                       double *h_out) {
  oracle_expert_ffn_fmt(0, H, I, gsz, qg, sg, qu, su, qd, sd, x, y, h_out);
}

/* The layer for S tokens given routing (idx, w):
 *   y[t] = sum_j w[t,j] * FFN_{idx[t,j]}(x_t)  (rank order)  +  FFN_shared(x_t).
 * Expert e's six parts are qg[e], sg[e], ... (pointer arrays of length E+1; entry E
 * is the shared expert, NULL when the layer has none).  Only experts that the
 * routing names need non-NULL pointers.  Every expert is in format fmt (R6). */
/* bf16_mask (optional, [E + 1], entry E the shared expert): experts computed with
 * bf16 operands (R8); NULL or all zero is the exact layer.  Not combined with R7. */
int oracle_moe_ffn_mask(int fmt, int act_int8, int S, int H, int E, int k, int I, int Is, int gsz, int x_is_bf16,
                        const void *x, const int32_t *idx, const double *w, const uint8_t *const *qg,
                        const void *const *sg, const uint8_t *const *qu, const void *const *su,
                        const uint8_t *const *qd, const void *const *sd, const uint8_t *bf16_mask, double *y) {
  if (act_int8 && bf16_mask)
    for (int e = 0; e <= E; ++e)
      if (bf16_mask[e]) return -2;
  double *xt = malloc(sizeof(double) * H), *xb = malloc(sizeof(double) * H), *ye = malloc(sizeof(double) * H),
         *acc = malloc(sizeof(double) * H);
  float *x32 = malloc(sizeof(float) * H);
  int rc = 0;
  for (int t = 0; t < S && !rc; ++t) {
    for (int c = 0; c < H; ++c) xt[c] = x_at(x, x_is_bf16, (size_t)t * H + c);
    if (act_int8) { /* R7: every expert of the token sees the quantised input */
      for (int c = 0; c < H; ++c) x32[c] = (float)xt[c];  /* fp32 and bf16 inputs are exact in fp32 */
      oracle_quant_row(H, x32, NULL, xt);
    }
    for (int c = 0; c < H; ++c) xb[c] = bf16_of(xt[c]); /* R8 input (exact for bf16 inputs) */
    for (int c = 0; c < H; ++c) acc[c] = 0.0;
    for (int j = 0; j < k; ++j) {
      int e = idx[(size_t)t * k + j];
      if (e < 0 || e >= E || !qg[e] || !sg[e] || !qu[e] || !su[e] || !qd[e] || !sd[e]) { rc = -1; break; }
      const int b = bf16_mask && bf16_mask[e];
      expert_ffn_impl(fmt, act_int8, b, H, I, gsz, qg[e], sg[e], qu[e], su[e], qd[e], sd[e], b ? xb : xt, ye, NULL);
      for (int c = 0; c < H; ++c) acc[c] += w[(size_t)t * k + j] * ye[c];
    }
    if (rc) break;
    if (Is > 0) {
      if (!qg[E]) { rc = -1; break; }
      const int b = bf16_mask && bf16_mask[E];
      expert_ffn_impl(fmt, act_int8, b, H, Is, gsz, qg[E], sg[E], qu[E], su[E], qd[E], sd[E], b ? xb : xt, ye, NULL);
      for (int c = 0; c < H; ++c) acc[c] += ye[c];
    }
    for (int c = 0; c < H; ++c) y[(size_t)t * H + c] = acc[c];
  }
  free(xt); free(xb); free(ye); free(acc); free(x32);
  return rc;
}

int oracle_moe_ffn_mode(int fmt, int act_int8, int S, int H, int E, int k, int I, int Is, int gsz, int x_is_bf16,
                        const void *x, const int32_t *idx, const double *w, const uint8_t *const *qg,
                        const void *const *sg, const uint8_t *const *qu, const void *const *su,
                        const uint8_t *const *qd, const void *const *sd, double *y) {
  return oracle_moe_ffn_mask(fmt, act_int8, S, H, E, k, I, Is, gsz, x_is_bf16, x, idx, w, qg, sg, qu, su, qd, sd,
                             NULL, y);
}

int oracle_moe_ffn_fmt(int fmt, int S, int H, int E, int k, int I, int Is, int gsz, int x_is_bf16, const void *x,
                       const int32_t *idx, const double *w, const uint8_t *const *qg, const void *const *sg,
                       const uint8_t *const *qu, const void *const *su, const uint8_t *const *qd,
                       const void *const *sd, double *y) {
  return oracle_moe_ffn_mode(fmt, 0, S, H, E, k, I, Is, gsz, x_is_bf16, x, idx, w, qg, sg, qu, su, qd, sd, y);
}

int oracle_moe_ffn(int S, int H, int E, int k, int I, int Is, int gsz, int x_is_bf16, const void *x,
                   const int32_t *idx, const double *w, const uint8_t *const *qg, const uint16_t *const *sg,
                   const uint8_t *const *qu, const uint16_t *const *su, const uint8_t *const *qd,
                   const uint16_t *const *sd, double *y) {
  return oracle_moe_ffn_fmt(0, S, H, E, k, I, Is, gsz, x_is_bf16, x, idx, w, qg, (const void *const *)sg, qu,
                            (const void *const *)su, qd, (const void *const *)sd, y);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads of the parallel loops from now on (the CPU-baseline timing runs the
 * oracle on one thread and on all of them). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
