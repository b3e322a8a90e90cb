/*
 * Seeded, counter-based generator of the synthetic inputs.
 *
 * This file holds no arithmetic of the MoE layer itself: it only draws the
 * input tensors (activations, router weight and bias, expert weights) that
 * both the GPU path and the CPU oracle consume, as the same host bytes.
 *
 * Definition (every element is computable on its own, so any slice can be
 * regenerated and the work splits freely over threads):
 *
 *   mix64(z)      = the SplitMix64 output function (Steele, Lea & Flood,
 *                   "Fast splittable pseudorandom number generators",
 *                   OOPSLA 2014): two xor-shift-multiply rounds and a final
 *                   xor-shift with the constants below.
 *   base(s, tau)  = mix64(mix64(s) ^ (tau * GAMMA))       one stream per tensor
 *   word(i)       = mix64(base + (i + 1) * GAMMA)          SplitMix64's i-th output
 *   uniform(i)    = ((word(i) >> 11) + 0.5) * 2^-53        in (0, 1)
 *   normal(i)     = sqrt(-2 ln uniform(2i)) * cos(2 pi uniform(2i + 1))
 *                   (Box & Muller 1958, cosine branch only)
 *
 * A value is formed in double (mean + std * normal), rounded to float by
 * the C cast (round to nearest even), and, for bf16 tensors, rounded from
 * float to bf16 with round-to-nearest-even on the upper 16 bits.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint64_t tensor) {
  return mix64(mix64(seed) ^ (tensor * GAMMA));
}

static inline double uniform_at(uint64_t base, uint64_t i) {
  uint64_t w = mix64(base + (i + 1) * GAMMA);
  return ((double)(w >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t base, uint64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = uniform_at(base, 2 * i);
  double u2 = uniform_at(base, 2 * i + 1);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)(u >> 16); /* inf/nan: not produced */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ jobs */

enum { OUT_F32 = 0, OUT_BF16 = 1 };
enum { DIST_NORMAL = 0, DIST_UNIFORM = 1 };

typedef struct {
  uint64_t base, row_base;
  int dist, out;
  double a, b;              /* normal: mean, std    uniform: lo, hi */
  int64_t begin, end;       /* element range handled by this worker */
  int64_t row_len;          /* >0: multiply by a per-row scale drawn from row_base */
  double row_lo, row_hi;    /* per-row scale ~ U(row_lo, row_hi) */
  void* dst;
} job_t;

static void* run_job(void* arg) {
  job_t* j = (job_t*)arg;
  for (int64_t i = j->begin; i < j->end; ++i) {
    double v = (j->dist == DIST_NORMAL) ? j->a + j->b * normal_at(j->base, (uint64_t)i)
                                        : j->a + (j->b - j->a) * uniform_at(j->base, (uint64_t)i);
    if (j->row_len > 0) {
      int64_t r = i / j->row_len;
      double c = j->row_lo + (j->row_hi - j->row_lo) * uniform_at(j->row_base, (uint64_t)r);
      v *= c;
    }
    float f = (float)v;
    if (j->out == OUT_F32)
      ((float*)j->dst)[i] = f;
    else
      ((uint16_t*)j->dst)[i] = f32_to_bf16_rne(f);
  }
  return NULL;
}

static int fill(job_t proto, int64_t n, int threads) {
  if (n <= 0) return 0;
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if (n < 65536) threads = 1;
  pthread_t tid[256];
  job_t jobs[256];
  int64_t chunk = (n + threads - 1) / threads;
  int started = 0;
  for (int t = 0; t < threads; ++t) {
    jobs[t] = proto;
    jobs[t].begin = (int64_t)t * chunk;
    jobs[t].end = jobs[t].begin + chunk < n ? jobs[t].begin + chunk : n;
    if (jobs[t].begin >= jobs[t].end) break;
    if (pthread_create(&tid[t], NULL, run_job, &jobs[t]) != 0) {
      run_job(&jobs[t]);
      tid[t] = 0;
    }
    started = t + 1;
  }
  for (int t = 0; t < started; ++t)
    if (tid[t]) pthread_join(tid[t], NULL);
  return 0;
}

/* ------------------------------------------------------------ public API */

/* n values ~ N(mean, std^2), as float32. */
int synth_normal_f32(uint64_t seed, uint64_t tensor, double mean, double std, float* dst,
                     int64_t n, int threads) {
  job_t j = {0};
  j.base = stream_base(seed, tensor);
  j.dist = DIST_NORMAL; j.out = OUT_F32; j.a = mean; j.b = std; j.dst = dst;
  return fill(j, n, threads);
}

/* n values ~ N(mean, std^2), float32 then bf16 (raw bits). */
int synth_normal_bf16(uint64_t seed, uint64_t tensor, double mean, double std, uint16_t* dst,
                      int64_t n, int threads) {
  job_t j = {0};
  j.base = stream_base(seed, tensor);
  j.dist = DIST_NORMAL; j.out = OUT_BF16; j.a = mean; j.b = std; j.dst = dst;
  return fill(j, n, threads);
}

/* rows x row_len values: N(mean, std^2) times a per-row factor ~ U(lo, hi)
 * drawn from the stream of tensor `row_tensor`; float32 then bf16. */
int synth_scaled_normal_bf16(uint64_t seed, uint64_t tensor, uint64_t row_tensor, double mean,
                             double std, double lo, double hi, uint16_t* dst, int64_t rows,
                             int64_t row_len, int threads) {
  job_t j = {0};
  j.base = stream_base(seed, tensor);
  j.row_base = stream_base(seed, row_tensor);
  j.dist = DIST_NORMAL; j.out = OUT_BF16; j.a = mean; j.b = std; j.dst = dst;
  j.row_len = row_len; j.row_lo = lo; j.row_hi = hi;
  return fill(j, rows * row_len, threads);
}

/* n values ~ U(lo, hi), float32. */
int synth_uniform_f32(uint64_t seed, uint64_t tensor, double lo, double hi, float* dst, int64_t n,
                      int threads) {
  job_t j = {0};
  j.base = stream_base(seed, tensor);
  j.dist = DIST_UNIFORM; j.out = OUT_F32; j.a = lo; j.b = hi; j.dst = dst;
  return fill(j, n, threads);
}

/* The first `m` entries of a seeded partial Fisher-Yates shuffle of [0, n):
 * for j in [0, m): r = j + floor(uniform(j) * (n - j)); swap(p[j], p[r]). */
int synth_choose(uint64_t seed, uint64_t tensor, int32_t n, int32_t m, int32_t* out) {
  if (n <= 0 || m < 0 || m > n) return 1;
  int32_t* p = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  if (!p) return 2;
  for (int32_t i = 0; i < n; ++i) p[i] = i;
  uint64_t base = stream_base(seed, tensor);
  for (int32_t j = 0; j < m; ++j) {
    int32_t r = j + (int32_t)floor(uniform_at(base, (uint64_t)j) * (double)(n - j));
    if (r >= n) r = n - 1;
    int32_t t = p[j]; p[j] = p[r]; p[r] = t;
  }
  memcpy(out, p, sizeof(int32_t) * (size_t)m);
  free(p);
  return 0;
}

/* Raw SplitMix64 words, for the generator's own known-answer tests. */
void synth_words(uint64_t seed, uint64_t tensor, uint64_t* dst, int64_t n) {
  uint64_t base = stream_base(seed, tensor);
  for (int64_t i = 0; i < n; ++i) dst[i] = mix64(base + (uint64_t)(i + 1) * GAMMA);
}

/* One SplitMix64 output for an explicit state, for checking mix64 against
 * the published reference outputs. */
uint64_t synth_splitmix64_next(uint64_t* state) {
  *state += GAMMA;
  return mix64(*state);
}

/* ------------------------------------------------------- fp8 (e4m3) rows */

/* OCP FP8 E4M3 ("e4m3fn"): sign, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent 0 holds the subnormals m * 2^-9; 0x7F/0xFF are NaN, so the
 * largest finite magnitude is 1.75 * 2^8 = 448.  Round to nearest, ties to
 * even mantissa; |v| <= 448 is required (the caller scales rows so). */
static uint8_t e4m3_rne(double v) {
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  const double a = fabs(v);
  if (a == 0.0) return sign;
  int ex;
  frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;                /* a in [2^e, 2^(e+1)) */
  int code;
  if (e < -6) {
    code = (int)nearbyint(ldexp(a, 9)); /* subnormal grid 2^-9; 8 is the smallest normal */
  } else {
    int m = (int)nearbyint((ldexp(a, -e) - 1.0) * 8.0);
    if (m == 8) { m = 0; ++e; }
    code = ((e + 7) << 3) | m;
  }
  if (code > 0x7E) code = 0x7E;  /* not reached for |v| <= 448 */
  return (uint8_t)(sign | code);
}

typedef struct {
  uint64_t base;
  double mean, std;
  int64_t row_begin, row_end, row_len;
  uint8_t* codes;
  float* scales;
} rows_job_t;

static void* run_rows(void* arg) {
  rows_job_t* j = (rows_job_t*)arg;
  float* row = (float*)malloc(sizeof(float) * (size_t)j->row_len);
  if (!row) return NULL;
  for (int64_t r = j->row_begin; r < j->row_end; ++r) {
    float amax = 0.0f;
    for (int64_t i = 0; i < j->row_len; ++i) {
      const int64_t idx = r * j->row_len + i;
      row[i] = (float)(j->mean + j->std * normal_at(j->base, (uint64_t)idx));
      const float m = fabsf(row[i]);
      if (m > amax) amax = m;
    }
    const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    j->scales[r] = scale;
    for (int64_t i = 0; i < j->row_len; ++i) {
      double q = (double)row[i] / (double)scale;
      if (q > 448.0) q = 448.0;
      if (q < -448.0) q = -448.0;
      j->codes[r * j->row_len + i] = e4m3_rne(q);
    }
  }
  free(row);
  return NULL;
}

/* rows x row_len weights drawn as synth_normal_bf16 draws them (same stream,
 * same element index), stored as e4m3 codes with one fp32 scale per row:
 * scale = max|row| / 448, code = e4m3(value / scale). */
int synth_normal_e4m3_rows(uint64_t seed, uint64_t tensor, double mean, double std,
                           uint8_t* codes, float* scales, int64_t rows, int64_t row_len,
                           int threads) {
  if (rows <= 0 || row_len <= 0) return 0;
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if (rows < threads) threads = (int)rows;
  pthread_t tid[256];
  rows_job_t jobs[256];
  const int64_t chunk = (rows + threads - 1) / threads;
  int started = 0;
  for (int t = 0; t < threads; ++t) {
    rows_job_t j = {stream_base(seed, tensor), mean, std, (int64_t)t * chunk, 0, row_len, codes,
                    scales};
    j.row_end = j.row_begin + chunk < rows ? j.row_begin + chunk : rows;
    if (j.row_begin >= j.row_end) break;
    jobs[t] = j;
    if (pthread_create(&tid[t], NULL, run_rows, &jobs[t]) != 0) {
      run_rows(&jobs[t]);
      tid[t] = 0;
    }
    started = t + 1;
  }
  for (int t = 0; t < started; ++t)
    if (tid[t]) pthread_join(tid[t], NULL);
  return 0;
}

/* The encoder alone, for tests: codes of n values (|v| <= 448). */
void synth_e4m3_encode(const double* v, int64_t n, uint8_t* codes) {
  for (int64_t i = 0; i < n; ++i) codes[i] = e4m3_rne(v[i]);
}
