/*
 * bwta_oracle.c - plain, slow, scalar CPU oracle for the binary-weight x
 * ternary-activation (BWTA) matrix product.
 *
 * TEST INFRASTRUCTURE ONLY.  This file exists to check the HIP library.  It is
 * loaded by the tests, by __graft_entry__.smoke() and by the CPU-baseline leg of
 * bench.py, and by nothing else.  It shares no code, header, table or constant
 * with the GPU library: everything below is written from the definitions.
 *
 * Source of the method: "BWTA: Accurate and Efficient Binarized Transformer by
 * Algorithm-Hardware Co-design" (Ding, Liu, Jin, Guo, Lu), Abstract: weights are
 * binary, activations are ternary with tiny values projected to zero, and the
 * product is computed by a bit-packed binary/ternary MatMul for linear and
 * attention operators; memory is one bit per weight and two per activation.
 * The pages fix no threshold, scale or reduction order.  The rules below are
 * the library's definition of those open points:
 *
 *   tree(v[0..n))  perfect pairwise fp32 tree over v zero-padded to the next
 *                  power of two P >= n; each level replaces (L[2i], L[2i+1]) by
 *                  fl32(L[2i] + L[2i+1]).
 *   binarize row   s = (w < 0) ? -1 : +1   (so sign(0) = sign(-0.0) = +1)
 *                  alpha_w = fl32(tree(|w|) / K)
 *   ternarize row  mu  = fl32(tree(|x|) / K);  thr = fl32(0.5 * mu)
 *                  t   = (|x| <= thr) ? 0 : (x < 0 ? -1 : +1)
 *                  nnz = #(t != 0)
 *                  alpha_a = nnz ? fl32(tree(t != 0 ? |x| : 0) / nnz) : 0
 *   packing        plane byte b, bit j (LSB = 0) holds k = 8b + j; a row holds
 *                  round_up(K, 64) / 8 bytes; bits k >= K are 0.
 *                  mask plane: t != 0; sign plane: value < 0.
 *   product        acc[m,n] = sum_k a[m,k] * b[n,k] in int32 (dense loop over
 *                  the unpacked values; no popcount anywhere in this file)
 *   epilogue       y = fl32((float)acc * fl32(alpha_a[m] * alpha_b[n]))
 *                  bf16(y) = round-to-nearest-even of the fp32 bits
 *   residual       (two binary planes per weight row; BiLLM page, Approach:
 *   binarize       salient weights get a residual, second-order binarization)
 *                  s1, alpha1 = binarize(w); r = fl32(w - alpha1 * s1), i.e.
 *                  w - alpha1 where s1 = +1 and w + alpha1 where s1 = -1;
 *                  s2, alpha2 = binarize(r)   so  w ~ alpha1 s1 + alpha2 s2
 *   residual       y = fl32(fl32((float)acc1 * fl32(alpha_a * alpha1))
 *   epilogue              + fl32((float)acc2 * fl32(alpha_a * alpha2)))
 *
 * Build: gcc -O2 -ffp-contract=off (no fast-math) so that every float
 * operation is one IEEE-754 binary32 operation, round-to-nearest-even.
 * Non-finite inputs are outside the contract: the calls that read floats return
 * a nonzero status for them.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_NONFINITE 1
#define ORACLE_ERR_ARGS 2
#define ORACLE_ERR_NOMEM 3

int64_t oracle_padded_k(int64_t K) { return (K + 63) / 64 * 64; }
int64_t oracle_row_bytes(int64_t K) { return oracle_padded_k(K) / 8; }

/* Perfect pairwise tree over v[0..n) zero-padded to a power of two. */
float oracle_tree_sum(const float* v, int64_t n) {
  if (n <= 0) return 0.0f;
  int64_t P = 1;
  while (P < n) P <<= 1;
  float* L = (float*)malloc((size_t)P * sizeof(float));
  if (!L) return NAN;
  for (int64_t i = 0; i < P; ++i) L[i] = (i < n) ? v[i] : 0.0f;
  for (int64_t width = P; width > 1; width >>= 1)
    for (int64_t i = 0; i < width / 2; ++i) L[i] = L[2 * i] + L[2 * i + 1];
  float r = L[0];
  free(L);
  return r;
}

/* bf16 bit patterns widen exactly to fp32 by a 16-bit left shift. */
void oracle_bf16_to_f32(const uint16_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u = (uint32_t)in[i] << 16;
    memcpy(&out[i], &u, 4);
  }
}

/* Round fp32 to bf16, nearest-even (inputs are finite). */
void oracle_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u;
    memcpy(&u, &in[i], 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    out[i] = (uint16_t)(u >> 16);
  }
}

/* Binary weights: W element (r, k) sits at W[r*stride_row + k*stride_k]. */
int oracle_binarize(const float* W, int64_t rows, int64_t K, int64_t stride_row,
                    int64_t stride_k, int8_t* s, float* alpha) {
  if (rows < 0 || K <= 0) return ORACLE_ERR_ARGS;
  float* a = (float*)malloc((size_t)K * sizeof(float));
  if (!a) return ORACLE_ERR_NOMEM;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t k = 0; k < K; ++k) {
      float w = W[r * stride_row + k * stride_k];
      if (!isfinite(w)) { free(a); return ORACLE_ERR_NONFINITE; }
      s[r * K + k] = (w < 0.0f) ? (int8_t)-1 : (int8_t)1;
      a[k] = fabsf(w);
    }
    alpha[r] = oracle_tree_sum(a, K) / (float)K;
  }
  free(a);
  return ORACLE_OK;
}

/* Residual (two-plane) binarization: the first plane and scale as
 * oracle_binarize, the second plane and scale those of the residual row
 * r = w - alpha1 * s1 (in fp32). */
int oracle_binarize_residual(const float* W, int64_t rows, int64_t K, int64_t stride_row,
                             int64_t stride_k, int8_t* s1, float* alpha1, int8_t* s2,
                             float* alpha2) {
  if (rows < 0 || K <= 0) return ORACLE_ERR_ARGS;
  int st = oracle_binarize(W, rows, K, stride_row, stride_k, s1, alpha1);
  if (st != ORACLE_OK) return st;
  float* res = (float*)malloc((size_t)K * sizeof(float));
  if (!res) return ORACLE_ERR_NOMEM;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t k = 0; k < K; ++k) {
      float w = W[r * stride_row + k * stride_k];
      res[k] = s1[r * K + k] < 0 ? w + alpha1[r] : w - alpha1[r];
    }
    st = oracle_binarize(res, 1, K, K, 1, s2 + r * K, alpha2 + r);
    if (st != ORACLE_OK) break;
  }
  free(res);
  return st;
}

/* Ternary activations, one row at a time; X row r starts at X + r*stride_row. */
int oracle_ternarize(const float* X, int64_t rows, int64_t K, int64_t stride_row,
                     int8_t* t, float* alpha, int32_t* nnz) {
  if (rows < 0 || K <= 0) return ORACLE_ERR_ARGS;
  float* a = (float*)malloc((size_t)K * sizeof(float));
  float* kept = (float*)malloc((size_t)K * sizeof(float));
  if (!a || !kept) { free(a); free(kept); return ORACLE_ERR_NOMEM; }
  for (int64_t r = 0; r < rows; ++r) {
    const float* x = X + r * stride_row;
    for (int64_t k = 0; k < K; ++k) {
      if (!isfinite(x[k])) { free(a); free(kept); return ORACLE_ERR_NONFINITE; }
      a[k] = fabsf(x[k]);
    }
    float mu = oracle_tree_sum(a, K) / (float)K;
    float thr = 0.5f * mu;
    int32_t count = 0;
    for (int64_t k = 0; k < K; ++k) {
      int8_t v;
      if (a[k] <= thr) v = 0;
      else v = (x[k] < 0.0f) ? (int8_t)-1 : (int8_t)1;
      t[r * K + k] = v;
      kept[k] = v ? a[k] : 0.0f;
      count += v ? 1 : 0;
    }
    nnz[r] = count;
    alpha[r] = count ? oracle_tree_sum(kept, K) / (float)count : 0.0f;
  }
  free(a);
  free(kept);
  return ORACLE_OK;
}

/* Pack one bit plane from unpacked values.  which = 0: bit = (v != 0) (mask);
 * which = 1: bit = (v < 0) (sign). */
int oracle_pack_plane(const int8_t* v, int64_t rows, int64_t K, int which, uint8_t* plane) {
  if (rows < 0 || K <= 0 || (which != 0 && which != 1)) return ORACLE_ERR_ARGS;
  int64_t rb = oracle_row_bytes(K);
  memset(plane, 0, (size_t)(rows * rb));
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k) {
      int8_t x = v[r * K + k];
      int bit = which == 0 ? (x != 0) : (x < 0);
      if (bit) plane[r * rb + k / 8] |= (uint8_t)(1u << (k % 8));
    }
  return ORACLE_OK;
}

/* acc[m*N + n] = sum_k A[m*K + k] * B[n*K + k], dense, int32. */
typedef struct {
  const int8_t* A;
  const int8_t* B;
  int64_t M, N, K, m0, m1;
  int32_t* acc;
} mm_job;

static void* mm_worker(void* p) {
  mm_job* j = (mm_job*)p;
  for (int64_t m = j->m0; m < j->m1; ++m)
    for (int64_t n = 0; n < j->N; ++n) {
      int32_t s = 0;
      const int8_t* a = j->A + m * j->K;
      const int8_t* b = j->B + n * j->K;
      for (int64_t k = 0; k < j->K; ++k) s += (int32_t)a[k] * (int32_t)b[k];
      j->acc[m * j->N + n] = s;
    }
  return NULL;
}

int oracle_matmul_i32(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t K,
                      int32_t* acc, int threads) {
  if (M < 0 || N < 0 || K <= 0) return ORACLE_ERR_ARGS;
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if (threads > M) threads = M > 0 ? (int)M : 1;
  pthread_t tid[256];
  mm_job jobs[256];
  int64_t per = (M + threads - 1) / threads;
  int started = 0;
  for (int i = 0; i < threads; ++i) {
    int64_t m0 = i * per, m1 = m0 + per > M ? M : m0 + per;
    jobs[i] = (mm_job){A, B, M, N, K, m0, m1, acc};
    if (m0 >= m1) continue;
    if (threads == 1 || pthread_create(&tid[i], NULL, mm_worker, &jobs[i]) != 0) {
      mm_worker(&jobs[i]);
      jobs[i].m0 = jobs[i].m1;  /* mark as done inline */
      continue;
    }
    tid[started] = tid[i];
    ++started;
  }
  for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
  return ORACLE_OK;
}

/* The same sums for a list of (m, n) pairs: out[i] = acc[mi[i], ni[i]]. */
int oracle_matmul_i32_pairs(const int8_t* A, const int8_t* B, int64_t K, const int64_t* mi,
                            const int64_t* ni, int64_t count, int32_t* out) {
  if (K <= 0 || count < 0) return ORACLE_ERR_ARGS;
  for (int64_t i = 0; i < count; ++i) {
    const int8_t* a = A + mi[i] * K;
    const int8_t* b = B + ni[i] * K;
    int32_t s = 0;
    for (int64_t k = 0; k < K; ++k) s += (int32_t)a[k] * (int32_t)b[k];
    out[i] = s;
  }
  return ORACLE_OK;
}

/* y[m*N + n] = fl32((float)acc * fl32(alpha_a[m] * alpha_b[n])). */
void oracle_scale(const int32_t* acc, const float* alpha_a, const float* alpha_b, int64_t M,
                  int64_t N, float* y) {
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      float s = alpha_a[m] * alpha_b[n];
      y[m * N + n] = (float)acc[m * N + n] * s;
    }
}

/* Epilogue of the two-plane product. */
void oracle_scale_residual(const int32_t* acc1, const int32_t* acc2, const float* alpha_a,
                           const float* alpha1, const float* alpha2, int64_t M, int64_t N,
                           float* y) {
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      float y1 = (float)acc1[m * N + n] * (alpha_a[m] * alpha1[n]);
      float y2 = (float)acc2[m * N + n] * (alpha_a[m] * alpha2[n]);
      y[m * N + n] = y1 + y2;
    }
}

/* Attention probabilities for the batched workload (input preparation between
 * the two attention products): z[m,n] = alpha_q[m] * alpha_k[n] * acc[m,n] /
 * sqrt(head_dim) in double, softmax over n with the row maximum subtracted, the
 * result rounded to fp32. */
void oracle_attention_probs(const int32_t* acc, const float* alpha_q, const float* alpha_k,
                            int64_t M, int64_t N, int64_t head_dim, float* P) {
  double inv = 1.0 / sqrt((double)head_dim);
  double* z = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
  for (int64_t m = 0; m < M; ++m) {
    double zmax = -INFINITY;
    for (int64_t n = 0; n < N; ++n) {
      z[n] = (double)alpha_q[m] * (double)alpha_k[n] * (double)acc[m * N + n] * inv;
      if (z[n] > zmax) zmax = z[n];
    }
    double sum = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      z[n] = exp(z[n] - zmax);
      sum += z[n];
    }
    for (int64_t n = 0; n < N; ++n) P[m * N + n] = (float)(z[n] / sum);
  }
  free(z);
}
