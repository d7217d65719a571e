/* Seeded synthetic input generator for the MoE-layer workloads.
 *
 * This file draws random numbers and encodes them into the input formats
 * (fp32, bf16 bits, fp16 bits, raw bytes).  It holds none of the MoE layer's
 * arithmetic: both the CPU oracle and the GPU library consume what it writes.
 *
 * Generator: the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), used counter-based:
 * draw(key, i) = mix64(key + (i + 1) * golden_gamma).  Every element depends only
 * on (key, index), so the output is identical for any thread count.
 * Normal variates: Box and Muller (1958), one variate per pair of uniforms.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t ctr) {
  return mix64(key + (ctr + 1) * GOLDEN_GAMMA);
}

/* uniform in [0, 1) with 53 random bits */
static inline double unif01(uint64_t r) { return (double)(r >> 11) * 0x1.0p-53; }
/* uniform in (0, 1] with 53 random bits (safe for log) */
static inline double unif01_open0(uint64_t r) { return (double)((r >> 11) + 1) * 0x1.0p-53; }

static inline double std_normal(uint64_t key, uint64_t i) {
  double u1 = unif01_open0(draw(key, 2 * i));
  double u2 = unif01(draw(key, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* double -> IEEE binary16 bits, round to nearest even (default FP environment). */
static uint16_t f64_to_f16_rne(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (isnan(a)) return (uint16_t)(sign | 0x7E00u);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
  if (a < 0x1p-14) { /* subnormal: a = m * 2^-24 */
    double m = nearbyint(a * 0x1p24);
    return (uint16_t)(sign | (uint16_t)m); /* m == 1024 encodes the smallest normal */
  }
  int e;
  (void)frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  double mant = nearbyint(ldexp(a, 11 - e)); /* in [1024, 2048] */
  int ex = e - 1;
  if (mant == 2048.0) { mant = 1024.0; ex += 1; }
  if (ex > 15) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)((ex + 15) << 10) | (uint16_t)(mant - 1024.0));
}

/* finite fp32 -> bf16 bits, round to nearest even */
static uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

uint64_t synth_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c, uint64_t d) {
  uint64_t k = mix64(seed + GOLDEN_GAMMA);
  k = mix64(k ^ (a * 0xD1B54A32D192ED03ULL + 1));
  k = mix64(k ^ (b * 0xAEF17502108EF2D9ULL + 2));
  k = mix64(k ^ (c * 0xF1357AEA2E62A9C5ULL + 3));
  k = mix64(k ^ (d * 0x9FB21C651E98DF25ULL + 4));
  return k;
}

/* n uniform random bytes (every nibble is then uniform on 0..15) */
void synth_fill_bytes(uint64_t key, uint64_t n, uint8_t* out) {
  int64_t nw = (int64_t)(n / 8);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nw; ++i) {
    uint64_t r = draw(key, (uint64_t)i);
    memcpy(out + 8 * i, &r, 8);
  }
  uint64_t rest = n - 8 * (uint64_t)nw;
  if (rest) {
    uint64_t r = draw(key, (uint64_t)nw);
    memcpy(out + 8 * nw, &r, rest);
  }
}

/* N(0, sigma^2) drawn in fp64, rounded to fp32 */
void synth_fill_normal_f32(uint64_t key, uint64_t n, double sigma, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = (float)(sigma * std_normal(key, (uint64_t)i));
}

/* N(0, sigma^2) drawn in fp64, rounded to fp32, then to bf16 (both RNE) */
void synth_fill_normal_bf16(uint64_t key, uint64_t n, double sigma, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i)
    out[i] = f32_to_bf16_rne((float)(sigma * std_normal(key, (uint64_t)i)));
}

/* |N(0, sigma^2)| drawn in fp64, rounded to fp16 bits */
void synth_fill_absnormal_f16(uint64_t key, uint64_t n, double sigma, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i)
    out[i] = f64_to_f16_rne(fabs(sigma * std_normal(key, (uint64_t)i)));
}

void synth_fill_normal_f64(uint64_t key, uint64_t n, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = std_normal(key, (uint64_t)i);
}

/* U(lo, hi) in fp64 */
void synth_fill_uniform_f64(uint64_t key, uint64_t n, double lo, double hi, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = lo + (hi - lo) * unif01(draw(key, (uint64_t)i));
}

/* uniform random permutation of 0..n-1 (Fisher-Yates) */
void synth_permutation(uint64_t key, int32_t n, int32_t* out) {
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    uint64_t j = draw(key, (uint64_t)i) % (uint64_t)(i + 1);
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}

/* encoders exposed so their rounding can be checked against numpy / torch */
void synth_encode_f16(uint64_t n, const double* in, uint16_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = f64_to_f16_rne(in[i]);
}
void synth_encode_bf16(uint64_t n, const float* in, uint16_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}
