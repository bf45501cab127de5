/*
 * oracle_sanitize_driver.c - runs the oracle's hand-derived pin cases as a
 * plain C program, so that tests/test_oracle_sanitize.py can build the oracle
 * with AddressSanitizer and UndefinedBehaviorSanitizer and execute every C
 * function of it at least once (out-of-bounds accesses, leaks, signed
 * overflow and misaligned accesses abort the run).
 *
 * TEST INFRASTRUCTURE ONLY: links oracle/bwta_oracle.c, nothing of the GPU
 * library.  The expected values are worked out by hand from the definitions at
 * the top of bwta_oracle.c (the BWTA page, Abstract, fixes the form; the
 * threshold 0.5 * mean|x| and the pairwise tree are the library's readings).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t oracle_padded_k(int64_t K);
int64_t oracle_row_bytes(int64_t K);
float oracle_tree_sum(const float* v, int64_t n);
void oracle_bf16_to_f32(const uint16_t* in, float* out, int64_t n);
void oracle_f32_to_bf16(const float* in, uint16_t* out, int64_t n);
int oracle_binarize(const float* W, int64_t rows, int64_t K, int64_t stride_row, int64_t stride_k,
                    int8_t* s, float* alpha);
int oracle_binarize_residual(const float* W, int64_t rows, int64_t K, int64_t stride_row,
                             int64_t stride_k, int8_t* s1, float* alpha1, int8_t* s2,
                             float* alpha2);
int oracle_ternarize(const float* X, int64_t rows, int64_t K, int64_t stride_row, int8_t* t,
                     float* alpha, int32_t* nnz);
int oracle_pack_plane(const int8_t* v, int64_t rows, int64_t K, int which, uint8_t* plane);
int oracle_matmul_i32(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t K,
                      int32_t* acc, int threads);
int oracle_matmul_i32_pairs(const int8_t* A, const int8_t* B, int64_t K, const int64_t* mi,
                            const int64_t* ni, int64_t count, int32_t* out);
void oracle_scale(const int32_t* acc, const float* alpha_a, const float* alpha_b, int64_t M,
                  int64_t N, float* y);
void oracle_scale_residual(const int32_t* acc1, const int32_t* acc2, const float* alpha_a,
                           const float* alpha1, const float* alpha2, int64_t M, int64_t N,
                           float* y);
void oracle_attention_probs(const int32_t* acc, const float* alpha_q, const float* alpha_k,
                            int64_t M, int64_t N, int64_t head_dim, float* P);

static int failures = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                    \
    }                                                                \
  } while (0)

/* Heap copies, so the sanitizer sees the exact extent of every buffer. */
static void* dup(const void* p, size_t n) {
  void* q = malloc(n);
  memcpy(q, p, n);
  return q;
}

int main(void) {
  /* Sizes: K = 65 needs two 64-bit words per row. */
  CHECK(oracle_padded_k(65) == 128 && oracle_row_bytes(65) == 16);
  CHECK(oracle_padded_k(64) == 64 && oracle_row_bytes(1) == 8);

  /* Tree order: fl32(2^24 + 1) = 2^24 (a tie, to even), but the right half
   * (1 + 1) = 2 survives, so the tree gives 2^24 + 2 where a left-to-right sum
   * gives 2^24.  With n = 3 the right half is (1 + 0) = 1, lost again. */
  {
    const float v0[4] = {16777216.0f, 1.0f, 1.0f, 1.0f};
    float* v = dup(v0, sizeof v0);
    CHECK(oracle_tree_sum(v, 4) == 16777218.0f);
    CHECK(oracle_tree_sum(v, 3) == 16777216.0f);
    free(v);
  }

  /* Ternarize x = [3, 1, 1, -3]: tree 8, mu 2, thr 1, |1| <= 1 drops. */
  {
    const float x0[4] = {3.0f, 1.0f, 1.0f, -3.0f};
    float* x = dup(x0, sizeof x0);
    int8_t* t = malloc(4);
    float a;
    int32_t nnz;
    CHECK(oracle_ternarize(x, 1, 4, 4, t, &a, &nnz) == 0);
    CHECK(t[0] == 1 && t[1] == 0 && t[2] == 0 && t[3] == -1);
    CHECK(nnz == 2 && a == 3.0f);
    uint8_t* mask = malloc(8);
    uint8_t* sign = malloc(8);
    CHECK(oracle_pack_plane(t, 1, 4, 0, mask) == 0);
    CHECK(oracle_pack_plane(t, 1, 4, 1, sign) == 0);
    CHECK(mask[0] == 0x09 && sign[0] == 0x08);
    for (int b = 1; b < 8; ++b) CHECK(mask[b] == 0 && sign[b] == 0);

    /* Weights [0.5, -0.25, -0.0, -0.25]: -0.0 maps to +1; alpha 0.25. */
    const float w0[4] = {0.5f, -0.25f, -0.0f, -0.25f};
    float* w = dup(w0, sizeof w0);
    int8_t* s = malloc(4);
    float aw;
    CHECK(oracle_binarize(w, 1, 4, 4, 1, s, &aw) == 0);
    CHECK(s[0] == 1 && s[1] == -1 && s[2] == 1 && s[3] == -1 && aw == 0.25f);
    uint8_t* ws = malloc(8);
    CHECK(oracle_pack_plane(s, 1, 4, 1, ws) == 0);
    CHECK(ws[0] == 0x0A);

    /* Product and epilogue: acc = 1 + 1 = 2, y = fl32(3 * 0.25) * 2 = 1.5. */
    int32_t* acc = malloc(sizeof(int32_t));
    CHECK(oracle_matmul_i32(t, s, 1, 1, 4, acc, 1) == 0);
    CHECK(acc[0] == 2);
    float* y = malloc(sizeof(float));
    oracle_scale(acc, &a, &aw, 1, 1, y);
    CHECK(y[0] == 1.5f);
    int64_t mi = 0, ni = 0;
    int32_t pair;
    CHECK(oracle_matmul_i32_pairs(t, s, 4, &mi, &ni, 1, &pair) == 0 && pair == 2);
    free(x); free(t); free(mask); free(sign); free(w); free(s); free(ws); free(acc); free(y);
  }

  /* Non-power-of-two K = 3, x = [1, 2, 4]: tree (1 + 2) + (4 + 0) = 7,
   * thr = fl32(7 / 3) / 2, so 1 drops; alpha = (2 + 4) / 2. */
  {
    const float x0[3] = {1.0f, 2.0f, 4.0f};
    float* x = dup(x0, sizeof x0);
    int8_t* t = malloc(3);
    float a;
    int32_t nnz;
    CHECK(oracle_ternarize(x, 1, 3, 3, t, &a, &nnz) == 0);
    CHECK(t[0] == 0 && t[1] == 1 && t[2] == 1 && nnz == 2 && a == 3.0f);
    uint8_t* mask = malloc(8);
    CHECK(oracle_pack_plane(t, 1, 3, 0, mask) == 0 && mask[0] == 0x06);
    free(x); free(t); free(mask);
  }

  /* An all-zero row: nnz 0, alpha 0.  A NaN: rejected. */
  {
    float* x = calloc(5, sizeof(float));
    int8_t* t = malloc(5);
    float a = -1.0f;
    int32_t nnz = -1;
    CHECK(oracle_ternarize(x, 1, 5, 5, t, &a, &nnz) == 0 && nnz == 0 && a == 0.0f);
    x[2] = NAN;
    CHECK(oracle_ternarize(x, 1, 5, 5, t, &a, &nnz) == 1);
    CHECK(oracle_ternarize(x, 1, 0, 5, t, &a, &nnz) == 2);
    free(x); free(t);
  }

  /* Bit planes of K = 65 (a row of 16 bytes): bit 64 lands in byte 8. */
  {
    int8_t* v = calloc(65, 1);
    v[0] = -1;
    v[64] = 1;
    uint8_t* p = malloc(16);
    CHECK(oracle_pack_plane(v, 1, 65, 0, p) == 0);
    CHECK(p[0] == 0x01 && p[8] == 0x01);
    CHECK(oracle_pack_plane(v, 1, 65, 1, p) == 0);
    CHECK(p[0] == 0x01 && p[8] == 0x00);
    free(v); free(p);
  }

  /* Columns (stride_k = ld): the columns of a 3 x 2 matrix. */
  {
    const float m0[6] = {1.0f, -2.0f, -3.0f, 4.0f, 5.0f, 0.0f};
    float* m = dup(m0, sizeof m0);
    int8_t* s = malloc(6);
    float* al = malloc(2 * sizeof(float));
    CHECK(oracle_binarize(m, 2, 3, 1, 2, s, al) == 0);
    CHECK(s[0] == 1 && s[1] == -1 && s[2] == 1 && s[3] == -1 && s[4] == 1 && s[5] == 1);
    CHECK(al[0] == 3.0f && al[1] == 2.0f); /* (1 + 3) + (5 + 0) = 9; (2 + 4) + 0 = 6 */
    free(m); free(s); free(al);
  }

  /* Two-plane residual: w = [2, -1, 1, -2], alpha1 = 6/4 = 1.5, residual
   * [0.5, 0.5, -0.5, -0.5], alpha2 = 0.5: w = 1.5 s1 + 0.5 s2 exactly. */
  {
    const float w0[4] = {2.0f, -1.0f, 1.0f, -2.0f};
    float* w = dup(w0, sizeof w0);
    int8_t* s1 = malloc(4);
    int8_t* s2 = malloc(4);
    float a1, a2;
    CHECK(oracle_binarize_residual(w, 1, 4, 4, 1, s1, &a1, s2, &a2) == 0);
    CHECK(a1 == 1.5f && a2 == 0.5f);
    CHECK(s1[0] == 1 && s1[1] == -1 && s1[2] == 1 && s1[3] == -1);
    CHECK(s2[0] == 1 && s2[1] == 1 && s2[2] == -1 && s2[3] == -1);
    const int32_t c1 = 3, c2 = -1;
    const float aa = 2.0f;
    float y;
    oracle_scale_residual(&c1, &c2, &aa, &a1, &a2, 1, 1, &y);
    CHECK(y == 8.0f); /* 3 * 3 + (-1) * 1 */
    free(w); free(s1); free(s2);
  }

  /* bf16: exact widening, round to nearest even on ties. */
  {
    const uint16_t h0[2] = {0x3F80, 0xC000};
    uint16_t* h = dup(h0, sizeof h0);
    float* f = malloc(2 * sizeof(float));
    oracle_bf16_to_f32(h, f, 2);
    CHECK(f[0] == 1.0f && f[1] == -2.0f);
    uint32_t bits[3] = {0x3F808000u, 0x3F818000u, 0x3F808001u};
    float* g = malloc(3 * sizeof(float));
    memcpy(g, bits, sizeof bits);
    uint16_t* o = malloc(3 * sizeof(uint16_t));
    oracle_f32_to_bf16(g, o, 3);
    CHECK(o[0] == 0x3F80 && o[1] == 0x3F82 && o[2] == 0x3F81);
    free(h); free(f); free(g); free(o);
  }

  /* Threaded product equals the single-thread one (rows split over threads,
   * more threads than rows included). */
  {
    const int64_t M = 7, N = 5, K = 100;
    int8_t* A = malloc(M * K);
    int8_t* B = malloc(N * K);
    for (int64_t i = 0; i < M * K; ++i) A[i] = (int8_t)((i * 7 + 3) % 3 - 1);
    for (int64_t i = 0; i < N * K; ++i) B[i] = (int8_t)((i * 5) % 2 ? -1 : 1);
    int32_t* c1 = malloc(M * N * sizeof(int32_t));
    int32_t* c3 = malloc(M * N * sizeof(int32_t));
    int32_t* c9 = malloc(M * N * sizeof(int32_t));
    CHECK(oracle_matmul_i32(A, B, M, N, K, c1, 1) == 0);
    CHECK(oracle_matmul_i32(A, B, M, N, K, c3, 3) == 0);
    CHECK(oracle_matmul_i32(A, B, M, N, K, c9, 9) == 0);
    CHECK(memcmp(c1, c3, M * N * sizeof(int32_t)) == 0);
    CHECK(memcmp(c1, c9, M * N * sizeof(int32_t)) == 0);
    free(A); free(B); free(c1); free(c3); free(c9);
  }

  /* Softmax of equal scores is uniform; one dominant score takes almost all. */
  {
    int32_t* acc = calloc(8, sizeof(int32_t));
    float* aq = malloc(2 * sizeof(float));
    float* ak = malloc(4 * sizeof(float));
    for (int i = 0; i < 2; ++i) aq[i] = 1.0f;
    for (int i = 0; i < 4; ++i) ak[i] = 1.0f;
    acc[4] = 1000;
    float* P = malloc(8 * sizeof(float));
    oracle_attention_probs(acc, aq, ak, 2, 4, 4, P);
    for (int n = 0; n < 4; ++n) CHECK(P[n] == 0.25f);
    CHECK(P[4] == 1.0f && P[5] == 0.0f);
    free(acc); free(aq); free(ak); free(P);
  }

  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle pins ok\n");
  return 0;
}
