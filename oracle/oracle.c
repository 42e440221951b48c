/*
 * oracle.c -- plain CPU reference of the W4A16 weight-only GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library. It shares no code, header,
 * table or helper with the GPU library; the two meet only through the arrays
 * of the seeded input generator.
 *
 * What it computes. The W4A16 scheme keeps weights in 4-bit storage and the
 * activations in 16-bit floating point (kongchang.com page, section "What
 * Exactly Is This Stack"). A decode step reads each weight matrix once and
 * multiplies it by the activation rows of every stream in the batch
 * (ai.satyajit.si page, section "One weight read, shared by every stream").
 * The 4-bit checkpoint is group-wise integer, one scale per group of weights
 * (same page, section "What one more stream costs on this model"):
 *
 *   w[n][k] = q[n][k] * s[n][floor(k/g)]                         (dequantize)
 *   y[m][n] = sum_{k=0}^{K-1} x[m][k] * w[n][k]                   (accumulate)
 *
 * with q in {-8..7}, s fp16, x bf16, g the group size. Both steps are done in
 * IEEE double: w is exact (at most 4 + 11 significant bits), each product
 * x*w is exact (8 + 15 <= 53 bits), and the sum runs in increasing k, so
 * the only rounding is that of the double additions. Output stays in double.
 *
 * The packed format (a reading of the pages, which say nothing about it).
 * Logical words: word j of output column n holds the codes of k = 8j..8j+7,
 * code of k = 8j+i in bits 4i..4i+3 as 4-bit two's complement (q & 0xF);
 * unpacking a code c gives ((c ^ 8) - 8). Device arrangement: columns are
 * taken in blocks of 16 (the last block padded with zero codes and zero
 * scales), and each (column block b, group t) tile of 16 columns x g weights
 * is stored contiguously as 64 lanes of g/32 consecutive words: lane l holds,
 * for column 16b + (l mod 16), the g/32 logical words that start at word
 * t*(g/8) + (l div 16)*(g/32). Tiles are ordered block-major, then by group.
 * Within a stored word the eight codes are interleaved: the code of
 * k = 8j+i sits in nibble (i div 2) + 4 (i mod 2), so nibbles 0..3 hold the
 * even k and nibbles 4..7 the odd k (nibbles v and v+4 are then codes 2v and
 * 2v+1, the two 16-bit halves of one register after a shift and a mask).
 * Scales are stored as [block][group][16]: entry (b, t, c) = s[16b + c][t].
  */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- number decoding (bf16 and fp16 bit patterns to double) ---- */

/* bf16 is the top half of an IEEE binary32. (Internal copies of the two
 * decoders are static, so that the compiler can inline them into the GEMM's
 * loops; the exported names below only forward to them.) */
static double bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double oracle_bf16_to_f64(uint16_t b) { return bf16_to_f64(b); }

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double fp16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1F;
  int frac = h & 0x3FF;
  double v;
  if (expo == 0) {
    v = ldexp((double)frac, -24);                 /* zero or subnormal */
  } else if (expo == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + frac), expo - 25);  /* 1.frac * 2^(expo-15) */
  }
  return sign ? -v : v;
}

double oracle_fp16_to_f64(uint16_t h) { return fp16_to_f64(h); }

/* ---- the GEMM ---- */

typedef struct {
  const uint16_t* x;
  const int8_t* q;
  const uint16_t* s;
  double* y;
  int M, N, K, group;
  int n0, n1;
} oracle_job;

/* Returns 0, or 1 if the column buffer could not be allocated. */
static int oracle_columns(const oracle_job* j) {
  const int K = j->K, G = K / j->group;
  double* w = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
  if (!w) return 1;
  for (int n = j->n0; n < j->n1; ++n) {
    /* dequantize column n: w[k] = q[n][k] * s[n][floor(k / g)] */
    const int8_t* qn = j->q + (size_t)n * K;
    const uint16_t* sn = j->s + (size_t)n * G;
    for (int k = 0; k < K; ++k) w[k] = (double)qn[k] * fp16_to_f64(sn[k / j->group]);
    /* accumulate: y[m][n] = sum_k x[m][k] * w[k], increasing k */
    for (int m = 0; m < j->M; ++m) {
      const uint16_t* xm = j->x + (size_t)m * K;
      double acc = 0.0;
      for (int k = 0; k < K; ++k) acc += bf16_to_f64(xm[k]) * w[k];
      j->y[(size_t)m * j->N + n] = acc;
    }
  }
  free(w);
  return 0;
}

static void* oracle_thread(void* p) {
  return (void*)(intptr_t)oracle_columns((const oracle_job*)p);
}

/*
 * y[M][N] (double) = x[M][K] (bf16 bits) times dequant(q[N][K] int8, s[N][K/group] fp16 bits).
 * Threads split the output columns; each dot product is summed by one thread
 * in increasing k, so the result does not depend on the thread count.
 * Returns 0; 1 on invalid arguments (nothing written); 2 if memory ran out.
 */
int oracle_gemm_f64(const uint16_t* x, const int8_t* q, const uint16_t* s, double* y,
                    int M, int N, int K, int group, int nthreads) {
  if (M < 0 || N < 0 || K < 0 || group <= 0 || K % group != 0) return 1;
  if ((M > 0 && N > 0) && (!y || (K > 0 && (!x || !q || !s)))) return 1;
  if (M == 0 || N == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > N) nthreads = N;
  oracle_job jobs[256];
  pthread_t th[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (oracle_job){x, q, s, y, M, N, K, group,
                           (int)((long long)N * t / nthreads),
                           (int)((long long)N * (t + 1) / nthreads)};
  }
  int started = 0, rc = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, oracle_thread, &jobs[t]) != 0) break;
    started = t;
  }
  rc |= oracle_columns(&jobs[0]);
  for (int t = 1; t <= started; ++t) {
    void* r = NULL;
    pthread_join(th[t], &r);
    rc |= (int)(intptr_t)r;
  }
  for (int t = started + 1; t < nthreads; ++t) rc |= oracle_columns(&jobs[t]);
  return rc ? 2 : 0;
}

/* ---- the packed format ---- */

/* Nibble of the stored word that holds the code of k = 8j + i. */
static int oracle_nibble(int i) { return i / 2 + 4 * (i % 2); }

/* Stored word j of column n (n < N), from the codes q[n][8j .. 8j+7]. */
static uint32_t oracle_stored_word(const int8_t* q, int K, int n, int j) {
  uint32_t word = 0;
  for (int i = 0; i < 8; ++i) {
    uint32_t code = (uint32_t)(q[(size_t)n * K + 8 * j + i] & 0xF);
    word |= code << (4 * oracle_nibble(i));
  }
  return word;
}

static int oracle_pack_shape_ok(int N, int K, int group) {
  return N >= 0 && K >= 0 && group > 0 && group % 32 == 0 && K % group == 0;
}

/* Number of 16-column blocks. */
static int oracle_blocks(int N) { return (N + 15) / 16; }

/*
 * Pack q[N][K] (int8, each in -8..7) and s[N][K/group] (fp16 bits) into the
 * device arrangement: qweight holds blocks*16*K/8 words, sp holds
 * blocks*(K/group)*16 fp16 values. Returns 0; 1 (nothing written) if the shape
 * is invalid (group % 32, K % group) or a code is out of range.
 */
int oracle_pack(const int8_t* q, const uint16_t* s, uint32_t* qweight, uint16_t* sp,
                int N, int K, int group) {
  if (!oracle_pack_shape_ok(N, K, group)) return 1;
  for (size_t i = 0; i < (size_t)N * K; ++i)
    if (q[i] < -8 || q[i] > 7) return 1;
  const int B = oracle_blocks(N), G = K / group, wpl = group / 32;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < G; ++t) {
      for (int l = 0; l < 64; ++l) {
        const int n = 16 * b + l % 16;
        for (int w = 0; w < wpl; ++w) {
          const int j = t * (group / 8) + (l / 16) * wpl + w;
          const size_t dst = (((size_t)b * G + t) * 64 + l) * wpl + w;
          qweight[dst] = n < N ? oracle_stored_word(q, K, n, j) : 0u;
        }
      }
      for (int c = 0; c < 16; ++c) {
        const int n = 16 * b + c;
        sp[((size_t)b * G + t) * 16 + c] = n < N ? s[(size_t)n * G + t] : (uint16_t)0;
      }
    }
  return 0;
}

/* Inverse of the weight half of oracle_pack: device words -> q[N][K]. */
int oracle_unpack(const uint32_t* qweight, int8_t* q, int N, int K, int group) {
  if (!oracle_pack_shape_ok(N, K, group)) return 1;
  const int G = K / group, wpl = group / 32;
  for (int n = 0; n < N; ++n) {
    const int b = n / 16, c = n % 16;
    for (int j = 0; j < K / 8; ++j) {
      const int t = j / (group / 8), r = j % (group / 8);
      const int l = (r / wpl) * 16 + c, w = r % wpl;
      const uint32_t word = qweight[(((size_t)b * G + t) * 64 + l) * wpl + w];
      for (int i = 0; i < 8; ++i) {
        const int code = (int)((word >> (4 * oracle_nibble(i))) & 0xF);
        q[(size_t)n * K + 8 * j + i] = (int8_t)((code ^ 8) - 8);
      }
    }
  }
  return 0;
}

/* ---- W4A8: int8 activations (per-row scale) times int4 weights ---- */
/*
 * The step past the bend: once the rows' arithmetic is the bottleneck, only
 * cheaper arithmetic raises the rate (ai.satyajit.si page, section "What one
 * more stream costs on this model"). Here the activations are quantized to
 * int8 with one scale per row, so that the products of codes are integers.
 *
 * Quantization of row m (a reading: the pages give no formula). All steps in
 * IEEE binary32 with round to nearest even, in this order:
 *   a      = max_k |x[m][k]|                       (exact: bf16 values)
 *   a == 0: sx[m] = 0 and every xq[m][k] = 0
 *   inv    = 127 / a                               (one rounding)
 *   t      = x[m][k] * inv                         (one rounding)
 *   xq     = nearest integer to t, ties to even, clamped to [-127, 127]
 *   sx[m]  = a / 127                               (one rounding)
 * GEMM: the integer sum per group is exact, the scaling is done in double:
 *   acc[m][n][t] = sum_{k in group t} xq[m][k] * q[n][k]        (exact)
 *   y[m][n]      = sx[m] * sum_t s[n][t] * acc[m][n][t]         (double, increasing t)
 */

/* Round a binary32 value to the nearest integer, ties to even. */
static float oracle_rne_int(float t) {
  const float f = floorf(t);
  const float d = t - f; /* exact: t and f are close binary32 values */
  if (d > 0.5f) return f + 1.0f;
  if (d < 0.5f) return f;
  return fmodf(f, 2.0f) == 0.0f ? f : f + 1.0f;
}

/*
 * Quantize x[M][K] (bf16 bits) row by row: xq[M][K] int8 (natural k order)
 * and sx[M] (binary32). Returns 0; 1 on invalid arguments (nothing written).
 */
int oracle_quantize_rows(const uint16_t* x, int8_t* xq, float* sx, int M, int K) {
  if (M < 0 || K < 0 || (M > 0 && K > 0 && (!x || !xq)) || (M > 0 && !sx)) return 1;
  for (int m = 0; m < M; ++m) {
    const uint16_t* xm = x + (size_t)m * K;
    float a = 0.0f;
    for (int k = 0; k < K; ++k) {
      const float v = fabsf((float)oracle_bf16_to_f64(xm[k]));
      if (v > a) a = v;
    }
    if (a == 0.0f) {
      sx[m] = 0.0f;
      for (int k = 0; k < K; ++k) xq[(size_t)m * K + k] = 0;
      continue;
    }
    volatile float inv = 127.0f / a;
    for (int k = 0; k < K; ++k) {
      volatile float t = (float)oracle_bf16_to_f64(xm[k]) * inv;
      float r = oracle_rne_int(t);
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      xq[(size_t)m * K + k] = (int8_t)r;
    }
    volatile float s = a / 127.0f;
    sx[m] = s;
  }
  return 0;
}

/*
 * y[M][N] (double) = W4A8 product of xq[M][K] (int8), sx[M] (binary32),
 * q[N][K] (int8 in -8..7) and s[N][K/group] (fp16 bits), as above.
 * Returns 0; 1 on invalid arguments.
 */
int oracle_gemm_w4a8(const int8_t* xq, const float* sx, const int8_t* q, const uint16_t* s,
                     double* y, int M, int N, int K, int group) {
  if (M < 0 || N < 0 || K < 0 || group <= 0 || K % group != 0) return 1;
  if (M == 0 || N == 0) return 0;
  if (!y || !sx || (K > 0 && (!xq || !q || !s))) return 1;
  const int G = K / group;
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n) {
      double sum = 0.0;
      for (int t = 0; t < G; ++t) {
        long long acc = 0;
        for (int k = t * group; k < (t + 1) * group; ++k)
          acc += (long long)xq[(size_t)m * K + k] * (long long)q[(size_t)n * K + k];
        sum += oracle_fp16_to_f64(s[(size_t)n * G + t]) * (double)acc;
      }
      y[(size_t)m * N + n] = (double)sx[m] * sum;
    }
  return 0;
}

/*
 * Device arrangement of quantized activations (a reading, chosen to match
 * the weights' stored words): row-major [M][K] int8, with each aligned block
 * of 16 consecutive k stored in the order of the codes of two stored words,
 * low nibbles then high nibbles: k offsets 0,4,1,5,2,6,3,7, 8,12,9,13,
 * 10,14,11,15. Group sums xsum[M][K/group] (int32) of the codes.
 */
static int oracle_xq_offset(int j) {
  static const int order[16] = {0, 4, 1, 5, 2, 6, 3, 7, 8, 12, 9, 13, 10, 14, 11, 15};
  return order[j];
}

int oracle_arrange_xq(const int8_t* xq, int8_t* out, int* xsum, int M, int K, int group) {
  if (M < 0 || K < 0 || K % 16 != 0 || group <= 0 || K % group != 0) return 1;
  for (int m = 0; m < M; ++m) {
    for (int b = 0; b < K / 16; ++b)
      for (int j = 0; j < 16; ++j)
        out[(size_t)m * K + 16 * b + j] = xq[(size_t)m * K + 16 * b + oracle_xq_offset(j)];
    for (int t = 0; t < K / group; ++t) {
      int acc = 0;
      for (int k = t * group; k < (t + 1) * group; ++k) acc += xq[(size_t)m * K + k];
      xsum[(size_t)m * (K / group) + t] = acc;
    }
  }
  return 0;
}
