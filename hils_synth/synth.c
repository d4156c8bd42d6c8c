/*
 * Seeded, counter-based synthetic input generator.
 *
 * This file holds no attention arithmetic.  It fills host buffers with
 * pseudo-random numbers that both sides of a parity check receive: the HIP
 * library (after an upload) and the float64 CPU oracle.  Every element is a
 * pure function of (seed, stream, element index), so results do not depend
 * on the number of threads.
 *
 * Definition
 *   mix(x)     SplitMix64 output function (Steele, Lea and Flood, "Fast
 *              splittable pseudorandom number generators", OOPSLA 2014):
 *                z = x + 0x9E3779B97F4A7C15
 *                z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
 *                z = (z ^ (z >> 27)) * 0x94D049BB133111EB
 *                return z ^ (z >> 31)
 *   key        = mix(mix(seed) ^ stream)
 *   word(i)    = mix(key + i)                         (64-bit wrap-around)
 *   normals    elements 2p and 2p+1 come from one Box-Muller pair
 *              (Box and Muller, Ann. Math. Stat. 29, 1958):
 *                u1 = ((word(2p) >> 11) + 1) * 2^-53      in (0, 1]
 *                u2 =  (word(2p+1) >> 11)    * 2^-53      in [0, 1)
 *                r  = sqrt(-2 ln u1)
 *                z[2p] = r cos(2 pi u2),  z[2p+1] = r sin(2 pi u2)
 *              value = mean + std * z, computed in double.
 *   uniforms   u(i) = (word(i) >> 11) * 2^-53, value = lo + (hi - lo) * u.
 *   storage    f64 as is; f32 by C's round-to-nearest cast; bf16 as the
 *              round-to-nearest-even of that f32 to 8 significant bits.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

enum { OUT_BF16 = 0, OUT_F32 = 1, OUT_F64 = 2 };

static inline uint64_t mix(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix(mix(seed) ^ stream);
}

static inline uint16_t f32_to_bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) /* inf / nan: keep class */
    return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

static inline void store(void *out, int type, uint64_t i, double v) {
  if (type == OUT_F64) {
    ((double *)out)[i] = v;
  } else if (type == OUT_F32) {
    ((float *)out)[i] = (float)v;
  } else {
    ((uint16_t *)out)[i] = f32_to_bf16_bits((float)v);
  }
}

uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t index) {
  return mix(stream_key(seed, stream) + index);
}

typedef struct {
  uint64_t key, lo, hi; /* element range [lo, hi) */
  double a, b;          /* normal: mean, std; uniform: lo, hi */
  int type, kind;       /* kind 0 normal, 1 uniform */
  void *out;
} job_t;

static void *run_job(void *arg) {
  const job_t *j = (const job_t *)arg;
  const double two_pi = 6.283185307179586476925286766559;
  const double ulp53 = 1.0 / 9007199254740992.0; /* 2^-53 */
  if (j->kind == 1) {
    for (uint64_t i = j->lo; i < j->hi; ++i) {
      double u = (double)(mix(j->key + i) >> 11) * ulp53;
      store(j->out, j->type, i, j->a + (j->b - j->a) * u);
    }
    return 0;
  }
  for (uint64_t i = j->lo & ~1ULL; i < j->hi; i += 2) {
    double u1 = (double)((mix(j->key + i) >> 11) + 1) * ulp53;
    double u2 = (double)(mix(j->key + i + 1) >> 11) * ulp53;
    double r = sqrt(-2.0 * log(u1));
    double z0 = r * cos(two_pi * u2), z1 = r * sin(two_pi * u2);
    if (i >= j->lo) store(j->out, j->type, i, j->a + j->b * z0);
    if (i + 1 < j->hi) store(j->out, j->type, i + 1, j->a + j->b * z1);
  }
  return 0;
}

static void launch(job_t proto, uint64_t n, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((uint64_t)nthreads > n / 4096 + 1) nthreads = (int)(n / 4096 + 1);
  pthread_t th[256];
  job_t jobs[256];
  uint64_t per = (n + nthreads - 1) / nthreads;
  per = (per + 1) & ~1ULL; /* keep Box-Muller pairs inside one job */
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = proto;
    jobs[t].lo = (uint64_t)t * per;
    jobs[t].hi = jobs[t].lo + per < n ? jobs[t].lo + per : n;
    if (jobs[t].lo >= n) break;
    if (pthread_create(&th[t], 0, run_job, &jobs[t]) != 0) {
      run_job(&jobs[t]);
      th[t] = 0;
    }
    started = t + 1;
  }
  for (int t = 0; t < started; ++t)
    if (th[t]) pthread_join(th[t], 0);
}

/* Fill out[0..n) with normals of the given mean and standard deviation. */
void synth_normal(uint64_t seed, uint64_t stream, uint64_t n, double mean,
                  double std, int out_type, void *out, int nthreads) {
  job_t p = {stream_key(seed, stream), 0, 0, mean, std, out_type, 0, out};
  launch(p, n, nthreads);
}

/* Fill out[0..n) with uniforms on [lo, hi). */
void synth_uniform(uint64_t seed, uint64_t stream, uint64_t n, double lo,
                   double hi, int out_type, void *out, int nthreads) {
  job_t p = {stream_key(seed, stream), 0, 0, lo, hi, out_type, 1, out};
  launch(p, n, nthreads);
}
