/*
 * Seeded synthetic input generator for the 4-bit attention workloads.
 *
 * This file holds NO arithmetic of the attention method itself: it only draws
 * Gaussian noise, applies rotary position embedding (a precondition: the
 * per-channel rescale the method applies acts on post-RoPE Q and K), applies
 * per-channel outlier multipliers and mean offsets that shape the inputs like
 * LLM attention activations, and rounds once to IEEE binary16.  Both the CPU
 * oracle and the GPU path consume its output; neither shares any other code.
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), used counter-style: the k-th
 * 64-bit draw of stream `seed` is mix(seed + (k + 1) * 0x9E3779B97F4A7C15).
 * Uniforms take the top 53 bits.  Normals use the Box-Muller transform on the
 * pair of uniforms (u[2i], u[2i+1]): element 2i takes the cosine branch,
 * element 2i+1 the sine branch.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t sm64_draw(uint64_t seed, uint64_t k) {
  return sm64_mix(seed + (k + 1ull) * 0x9E3779B97F4A7C15ull);
}

/* uniform in [0, 1) with 53 random bits */
static inline double sm64_uniform(uint64_t seed, uint64_t k) {
  return (double)(sm64_draw(seed, k) >> 11) * (1.0 / 9007199254740992.0);
}

/* element i of the standard-normal stream `seed` */
static inline double sm64_normal(uint64_t seed, uint64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  uint64_t pair = i >> 1;
  double u1 = 1.0 - sm64_uniform(seed, 2 * pair); /* (0, 1] so log is finite */
  double u2 = sm64_uniform(seed, 2 * pair + 1);
  double r = sqrt(-2.0 * log(u1));
  return (i & 1) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
}

/* IEEE binary16 round-to-nearest-even from a double, in one rounding step. */
static uint16_t f16_from_f64(double x) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  double a = fabs(x);
  if (isnan(x)) return 0x7E00u;
  if (a >= 65520.0) return sign | 0x7C00u; /* rounds to infinity */
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: value = q * 2^-24, q in [0, 1024] */
    double q = a * 16777216.0;           /* exact scaling by 2^24 */
    double fl = floor(q), rem = q - fl;
    uint32_t m = (uint32_t)fl;
    if (rem > 0.5 || (rem == 0.5 && (m & 1u))) m++;
    return sign | (uint16_t)m; /* m == 1024 gives the smallest normal */
  }
  int e;
  double fr = frexp(a, &e); /* a = fr * 2^e, fr in [0.5, 1) */
  /* normal: a = 1.mmmmmmmmmm * 2^(e-1); mantissa with 10 fraction bits */
  double q = ldexp(fr, 11); /* in [1024, 2048) */
  double fl = floor(q), rem = q - fl;
  uint32_t m = (uint32_t)fl;
  if (rem > 0.5 || (rem == 0.5 && (m & 1u))) m++;
  int exp16 = e - 1 + 15;
  if (m == 2048u) { m = 1024u; exp16++; }
  if (exp16 >= 31) return sign | 0x7C00u;
  return sign | (uint16_t)((uint32_t)exp16 << 10) | (uint16_t)(m - 1024u);
}

uint16_t synth_f16_from_f64(double x) { return f16_from_f64(x); }

void synth_normal_f64(uint64_t seed, uint64_t first, int64_t n, double* out) {
  for (int64_t i = 0; i < n; i++) out[i] = sm64_normal(seed, first + (uint64_t)i);
}

void synth_uniform_f64(uint64_t seed, uint64_t first, int64_t n, double* out) {
  for (int64_t i = 0; i < n; i++) out[i] = sm64_uniform(seed, first + (uint64_t)i);
}

void synth_raw_u64(uint64_t seed, uint64_t first, int64_t n, uint64_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = sm64_draw(seed, first + (uint64_t)i);
}

/*
 * Fill x[B][H][N][d] (binary16 bits) with
 *   x = (RoPE_theta(noise))[.., j] * mult[h][j] + offset[h][j]
 * where noise element (b, h, p, j) is normal number ((b*H + h)*N + p)*d + j of
 * stream `seed`, RoPE is the rotate-half form pairing channels j and j + d/2
 * with angle (pos0 + p) * theta^(-2j/d) (theta <= 0 disables it), and
 * mult/offset are per (head, channel) arrays (NULL = 1 / 0).
 */
typedef struct {
  uint64_t seed;
  int64_t B, H, N, d, pos0;
  double theta;
  const double* mult;
  const double* offset;
  uint16_t* out;
  int64_t bh_begin, bh_end;
} synth_job;

static void* synth_worker(void* arg) {
  synth_job* jb = (synth_job*)arg;
  const int64_t N = jb->N, d = jb->d, H = jb->H;
  double* row = (double*)malloc(sizeof(double) * (size_t)d);
  double* inv_freq = (double*)malloc(sizeof(double) * (size_t)(d / 2 > 0 ? d / 2 : 1));
  for (int64_t j = 0; j < d / 2; j++) inv_freq[j] = pow(jb->theta, -2.0 * (double)j / (double)d);
  for (int64_t bh = jb->bh_begin; bh < jb->bh_end; bh++) {
    int64_t h = bh % H;
    for (int64_t p = 0; p < N; p++) {
      uint64_t base = (uint64_t)((bh * N + p) * d);
      for (int64_t j = 0; j < d; j++) row[j] = sm64_normal(jb->seed, base + (uint64_t)j);
      if (jb->theta > 0.0) {
        double pos = (double)(jb->pos0 + p);
        for (int64_t j = 0; j < d / 2; j++) {
          double ang = pos * inv_freq[j];
          double c = cos(ang), s = sin(ang);
          double x1 = row[j], x2 = row[j + d / 2];
          row[j] = x1 * c - x2 * s;
          row[j + d / 2] = x2 * c + x1 * s;
        }
      }
      uint16_t* o = jb->out + (size_t)((bh * N + p) * d);
      for (int64_t j = 0; j < d; j++) {
        double v = row[j];
        if (jb->mult) v *= jb->mult[h * d + j];
        if (jb->offset) v += jb->offset[h * d + j];
        o[j] = f16_from_f64(v);
      }
    }
  }
  free(row);
  free(inv_freq);
  return NULL;
}

int synth_tensor_f16(uint64_t seed, int64_t B, int64_t H, int64_t N, int64_t d, int64_t pos0,
                     double theta, const double* mult, const double* offset, uint16_t* out,
                     int threads) {
  if (B < 0 || H < 0 || N < 0 || d <= 0 || (d & 1)) return -1;
  int64_t total = B * H;
  if (total == 0 || N == 0) return 0;
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if (threads > total) threads = (int)total;
  pthread_t tid[256];
  synth_job jobs[256];
  for (int t = 0; t < threads; t++) {
    synth_job* jb = &jobs[t];
    jb->seed = seed; jb->B = B; jb->H = H; jb->N = N; jb->d = d; jb->pos0 = pos0;
    jb->theta = theta; jb->mult = mult; jb->offset = offset; jb->out = out;
    jb->bh_begin = total * t / threads;
    jb->bh_end = total * (t + 1) / threads;
    if (pthread_create(&tid[t], NULL, synth_worker, jb) != 0) {
      synth_worker(jb);
      tid[t] = 0;
    }
  }
  for (int t = 0; t < threads; t++)
    if (tid[t]) pthread_join(tid[t], NULL);
  return 0;
}
