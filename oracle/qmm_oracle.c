/*
 * qmm_oracle.c -- plain, slow, float64 CPU oracle for the affine group-quantized
 * matmul y = x . W^T.  TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and
 * the CPU-baseline leg of the bench may load it.  It shares no code, header or
 * table with the GPU library.
 *
 * Sources (the pages):
 *   [P1] "@mlx-bun/inference 0.0.0-stage -> 1.0.0" (diffend npm page 53)
 *        - affine-split-mma.ts, header comment: the operation is y = x . W^T over
 *          MLX affine 3- or 4-bit, group-64 weights.
 *        - affine-split-mma.ts, HEADER helper affine_unit: value v of a group is
 *          read from MLX's LSB-first bit stream and may straddle into the next
 *          32-bit word.
 *        - affine3-mma.ts, helper affine_q3 (bit = 3t, word = bit>>5, the low
 *          bits come from that word, the rest from the next one); kernel body:
 *          row n starts at byte n*K*3/8, scale/bias of (n, g) at n*(K/64)+g,
 *          weight = fma(scale, q, bias).
 *        - affine4-mma.ts, helper affine_q4 (4-bit values never straddle).
 *        - affine3-rows.ts header comment: same algebra as MLX,
 *          sum_g scale*sum q*x + bias*sum x.
 *
 * What is computed is the plain definition, in float64, with no blocking,
 * reordering or fusion:
 *   q(n,k)  = the `bits`-bit unsigned field at bit offset k*bits of row n's
 *             LSB-first bit stream (rows are K*bits/32 uint32 words long),
 *             gathered one bit at a time;
 *   W(n,k)  = scale(n, k/gs) * q(n,k) + bias(n, k/gs);
 *   y(m,n)  = sum_{k=0}^{K-1} x(m,k) * W(n,k), summed in ascending k.
 * Inputs are handed over already decoded to float64 (bf16 and f32 values are
 * exact in float64), so every product is exact and y carries only the
 * ascending-order rounding of K float64 additions.
 */
#include <stdint.h>
#include <stdlib.h>
#include <math.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)

static int args_ok(int bits, int64_t K, int64_t N, int64_t gs) {
  if (bits < 1 || bits > 8) return 0;
  if (K <= 0 || N <= 0 || gs <= 0) return 0;
  if (K % gs != 0) return 0;
  if ((K * bits) % 32 != 0) return 0; /* every row is a whole number of words */
  return 1;
}

/* One code, one bit at a time: bit i of the value is bit (k*bits + i) of the
 * row's stream; stream bit p lives in word p/32 at position p%32 (LSB first). */
static unsigned code_at(const uint32_t *row, int bits, int64_t k) {
  unsigned q = 0;
  for (int i = 0; i < bits; ++i) {
    int64_t p = k * (int64_t)bits + i;
    unsigned bit = (row[p >> 5] >> (p & 31)) & 1u;
    q |= bit << i;
  }
  return q;
}

/* codes[n*K + k] = q(n,k). */
int qmm_oracle_unpack(int bits, int64_t K, int64_t N, const uint32_t *w,
                      uint8_t *codes) {
  if (!args_ok(bits, K, N, 1) || !w || !codes) return ORACLE_BAD_ARG;
  const int64_t words = K * bits / 32;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k)
      codes[n * K + k] = (uint8_t)code_at(w + n * words, bits, k);
  return ORACLE_OK;
}

/* W(n, .) as float64 into wrow[K]. */
static void dequant_row(int bits, int64_t K, int64_t gs, const uint32_t *row,
                        const double *s, const double *b, double *wrow) {
  for (int64_t k = 0; k < K; ++k) {
    const double q = (double)code_at(row, bits, k);
    wrow[k] = s[k / gs] * q + b[k / gs];
  }
}

/* y[m*N + n] for all m < M, n < N.  Rows of W are independent, so they are
 * shared out over `threads` OpenMP threads; every y element is still one
 * thread's ascending-k sum, so the result does not depend on `threads`. */
int qmm_oracle_matmul(int bits, int64_t gs, int64_t K, int64_t N, int64_t M,
                      const double *x, const uint32_t *w, const double *scales,
                      const double *biases, double *y, int threads) {
  if (!args_ok(bits, K, N, gs) || M <= 0 || !x || !w || !scales || !biases || !y)
    return ORACLE_BAD_ARG;
  const int64_t words = K * bits / 32, G = K / gs;
  int bad = 0;
#pragma omp parallel num_threads(threads > 0 ? threads : 1)
  {
    double *wrow = (double *)malloc((size_t)K * sizeof(double));
    if (!wrow) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(static)
      for (int64_t n = 0; n < N; ++n) {
        dequant_row(bits, K, gs, w + n * words, scales + n * G, biases + n * G, wrow);
        for (int64_t m = 0; m < M; ++m) {
          double acc = 0.0;
          for (int64_t k = 0; k < K; ++k) acc += x[m * K + k] * wrow[k];
          y[m * N + n] = acc;
        }
      }
      free(wrow);
    }
  }
  return bad ? ORACLE_BAD_ARG : ORACLE_OK;
}

/* out[i] = y(ms[i], ns[i]) for `count` sampled output elements. */
int qmm_oracle_matmul_at(int bits, int64_t gs, int64_t K, int64_t N, int64_t M,
                         const double *x, const uint32_t *w, const double *scales,
                         const double *biases, int64_t count, const int64_t *ms,
                         const int64_t *ns, double *out) {
  if (!args_ok(bits, K, N, gs) || M <= 0 || count < 0) return ORACLE_BAD_ARG;
  const int64_t words = K * bits / 32, G = K / gs;
  double *wrow = (double *)malloc((size_t)K * sizeof(double));
  if (!wrow) return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < count; ++i) {
    const int64_t m = ms[i], n = ns[i];
    if (m < 0 || m >= M || n < 0 || n >= N) { free(wrow); return ORACLE_BAD_ARG; }
    dequant_row(bits, K, gs, w + n * words, scales + n * G, biases + n * G, wrow);
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += x[m * K + k] * wrow[k];
    out[i] = acc;
  }
  free(wrow);
  return ORACLE_OK;
}

/* The two factors of the acceptance bound: sum_k |x(m,k)| per activation row
 * and max_k |W(n,k)| per weight row. */
int qmm_oracle_bound_terms(int bits, int64_t gs, int64_t K, int64_t N, int64_t M,
                           const double *x, const uint32_t *w, const double *scales,
                           const double *biases, double *sum_abs_x,
                           double *max_abs_w) {
  if (!args_ok(bits, K, N, gs) || M <= 0) return ORACLE_BAD_ARG;
  const int64_t words = K * bits / 32, G = K / gs;
  for (int64_t m = 0; m < M; ++m) {
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += fabs(x[m * K + k]);
    sum_abs_x[m] = s;
  }
  double *wrow = (double *)malloc((size_t)K * sizeof(double));
  if (!wrow) return ORACLE_BAD_ARG;
  for (int64_t n = 0; n < N; ++n) {
    dequant_row(bits, K, gs, w + n * words, scales + n * G, biases + n * G, wrow);
    double mx = 0.0;
    for (int64_t k = 0; k < K; ++k) mx = fmax(mx, fabs(wrow[k]));
    max_abs_w[n] = mx;
  }
  free(wrow);
  return ORACLE_OK;
}
