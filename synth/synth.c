/*
 * synth.c -- seeded, counter-based synthetic inputs for the W4A16 GEMM.
 *
 * This module only draws numbers. It holds none of the GEMM's arithmetic: it
 * produces logical int4 weight codes (one int8 per weight), fp16 group scales
 * and bf16 activations, and both the CPU oracle and the GPU library consume
 * the same arrays. Every element is a pure function of (seed, tensor id,
 * element index), so any slice of any tensor can be regenerated on its own.
 *
 * Generator: SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), with the 64-bit finaliser
 * constants of its public reference implementation. The i-th output (i from
 * 0) of a generator whose state starts at `key` is mix(key + (i+1)*gamma).
 *
 * Distributions (the decode workloads: int4 codes uniform on [-8, 7], fp16
 * scales uniform on [0.005, 0.02], bf16 activations standard normal):
 *   q[n][k] = (r >> 60) - 8                    r = out(key_q, n*K + k)
 *   s[n][j] = RNE_fp16(0.005 + 0.015 * u)      u = (r >> 11) * 2^-53
 *   x[m][k] = RNE_bf16(sqrt(-2 ln u1) cos(2 pi u2))   (Box and Muller, 1958)
 *             u1 = ((r1 >> 11) + 1) * 2^-53, u2 = (r2 >> 11) * 2^-53,
 *             r1 = out(key_x, 2i), r2 = out(key_x, 2i+1), i = m*K + k
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

static uint64_t synth_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* i-th output of SplitMix64 started at state `key`. */
uint64_t synth_splitmix64(uint64_t key, uint64_t i) {
  return synth_mix(key + (i + 1) * SYNTH_GAMMA);
}

/* Stream key of one tensor: the tensor_id-th output of SplitMix64 seeded with `seed`. */
uint64_t synth_stream_key(uint64_t seed, uint64_t tensor_id) {
  return synth_splitmix64(seed, tensor_id);
}

/* Round a finite double to the nearest fp16, ties to even (IEEE 754 binary16). */
uint16_t synth_f64_to_fp16_rne(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  (void)frexp(a, &e);           /* a = f * 2^e, f in [0.5, 1) */
  int ue = e - 1;               /* a = 1.x * 2^ue */
  if (ue < -14) {               /* subnormal range: units of 2^-24 */
    double r = nearbyint(ldexp(a, 24));
    return (uint16_t)(sign | (uint16_t)r); /* r == 1024 lands on the smallest normal */
  }
  double r = nearbyint(ldexp(a, 10 - ue)); /* significand in [1024, 2048] */
  if (r == 2048.0) { r = 1024.0; ue += 1; }
  if (ue > 15) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)((ue + 15) << 10) | (uint16_t)(r - 1024.0));
}

/* Round a finite double to the nearest bf16, ties to even (8-bit significand, binary32 exponent). */
uint16_t synth_f64_to_bf16_rne(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  (void)frexp(a, &e);
  int ue = e - 1;
  if (ue < -126) {              /* subnormal range: units of 2^-133 */
    double r = nearbyint(ldexp(a, 133));
    return (uint16_t)(sign | (uint16_t)r);
  }
  double r = nearbyint(ldexp(a, 7 - ue)); /* significand in [128, 256] */
  if (r == 256.0) { r = 128.0; ue += 1; }
  if (ue > 127) return (uint16_t)(sign | 0x7F80u);
  return (uint16_t)(sign | (uint16_t)((ue + 127) << 7) | (uint16_t)(r - 128.0));
}

/* ---- work splitting over threads (rows of the output tensor) ---- */

typedef struct {
  int kind;          /* 0 = q, 1 = scales, 2 = x */
  double sigma;      /* x only: standard deviation (1 for the workloads) */
  uint64_t key;
  void* out;
  int64_t cols;      /* elements per row */
  int64_t r0, r1;    /* rows [r0, r1) of the full tensor, written from out[0] */
  int64_t t0, t1;    /* this thread's row range */
} synth_job;

static void synth_rows(const synth_job* j) {
  for (int64_t r = j->t0; r < j->t1; ++r) {
    int64_t base = (r - j->r0) * j->cols;
    for (int64_t c = 0; c < j->cols; ++c) {
      uint64_t i = (uint64_t)(r * j->cols + c);
      if (j->kind == 0) {
        uint64_t z = synth_splitmix64(j->key, i);
        ((int8_t*)j->out)[base + c] = (int8_t)((int)(z >> 60) - 8);
      } else if (j->kind == 1) {
        uint64_t z = synth_splitmix64(j->key, i);
        double u = (double)(z >> 11) * 0x1.0p-53;
        ((uint16_t*)j->out)[base + c] = synth_f64_to_fp16_rne(0.005 + 0.015 * u);
      } else {
        uint64_t z1 = synth_splitmix64(j->key, 2 * i);
        uint64_t z2 = synth_splitmix64(j->key, 2 * i + 1);
        double u1 = (double)((z1 >> 11) + 1) * 0x1.0p-53;
        double u2 = (double)(z2 >> 11) * 0x1.0p-53;
        double g = sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
        ((uint16_t*)j->out)[base + c] = synth_f64_to_bf16_rne(j->sigma * g);
      }
    }
  }
}

static void* synth_thread(void* p) {
  synth_rows((const synth_job*)p);
  return NULL;
}

static int synth_run(int kind, double sigma, uint64_t seed, uint64_t tensor_id, void* out,
                     int64_t cols, int64_t r0, int64_t r1, int nthreads) {
  if (!out || cols < 0 || r0 < 0 || r1 < r0) return 1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  int64_t rows = r1 - r0;
  if (rows < nthreads) nthreads = rows > 0 ? (int)rows : 1;
  synth_job jobs[64];
  pthread_t th[64];
  uint64_t key = synth_stream_key(seed, tensor_id);
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].kind = kind;
    jobs[t].sigma = sigma;
    jobs[t].key = key;
    jobs[t].out = out;
    jobs[t].cols = cols;
    jobs[t].r0 = r0;
    jobs[t].r1 = r1;
    jobs[t].t0 = r0 + rows * t / nthreads;
    jobs[t].t1 = r0 + rows * (t + 1) / nthreads;
  }
  int started = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, synth_thread, &jobs[t]) != 0) break;
    started = t;
  }
  synth_rows(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
  for (int t = started + 1; t < nthreads; ++t) synth_rows(&jobs[t]); /* threads that failed to start */
  return 0;
}

/* Rows [n0, n1) of the int4 codes q[N][K] (one int8 per weight, values -8..7). */
int synth_q(uint64_t seed, uint64_t tensor_id, int8_t* out, int64_t K, int64_t n0, int64_t n1,
            int nthreads) {
  return synth_run(0, 1.0, seed, tensor_id, out, K, n0, n1, nthreads);
}

/* Rows [n0, n1) of the fp16 group scales s[N][G] (bit patterns). */
int synth_scales(uint64_t seed, uint64_t tensor_id, uint16_t* out, int64_t G, int64_t n0,
                 int64_t n1, int nthreads) {
  return synth_run(1, 1.0, seed, tensor_id, out, G, n0, n1, nthreads);
}

/* Rows [m0, m1) of the bf16 activations x[M][K] (bit patterns). */
int synth_x(uint64_t seed, uint64_t tensor_id, uint16_t* out, int64_t K, int64_t m0, int64_t m1,
            int nthreads) {
  return synth_run(2, 1.0, seed, tensor_id, out, K, m0, m1, nthreads);
}

/* As synth_x, with standard deviation sigma: x[m][k] = RNE_bf16(sigma * g), g the
 * same Box-Muller normal (sigma = 1 gives synth_x's values). */
int synth_x_sigma(uint64_t seed, uint64_t tensor_id, uint16_t* out, int64_t K, int64_t m0,
                  int64_t m1, double sigma, int nthreads) {
  return synth_run(2, sigma, seed, tensor_id, out, K, m0, m1, nthreads);
}
