/*
 * bwta.h - C ABI of libbwta.so, the binary-weight x ternary-activation (BWTA)
 * matrix-product library for AMD Instinct MI355X (gfx950).
 *
 * The method is the one of "BWTA: Accurate and Efficient Binarized Transformer
 * by Algorithm-Hardware Co-design" (Ding, Liu, Jin, Guo, Lu), Abstract: weights
 * are binary, activations are ternary with tiny values projected to zero, both
 * are bit-packed (one bit per weight, two per activation), and binary/ternary
 * MatMuls serve the linear and the attention operators.  The page fixes no
 * threshold, scale or reduction order; this library defines them as follows.
 *
 * Definitions (every call below computes exactly these; all float operations
 * are IEEE-754 binary32, round to nearest even, no fused multiply-add):
 *
 *   tree(v[0..n))  perfect pairwise tree over v zero-padded to the next power
 *                  of two P >= n: each level replaces (L[2i], L[2i+1]) by
 *                  L[2i] + L[2i+1].
 *   binarize       s[k] = (w[k] < 0) ? -1 : +1   (so -0.0 and +0.0 give +1)
 *                  alpha_w = tree(|w|) / K
 *   ternarize      mu = tree(|x|) / K;  thr = 0.5f * mu
 *                  t[k] = (|x[k]| <= thr) ? 0 : (x[k] < 0 ? -1 : +1)
 *                  nnz = #{k : t[k] != 0}
 *                  alpha_a = nnz ? tree(t[k] != 0 ? |x[k]| : 0) / nnz : 0
 *   product        acc[m][n] = sum_k a[m][k] * b[n][k]  (int32, exact)
 *   epilogue       y = (float)acc * (alpha_a[m] * alpha_b[n]);  bf16 output is
 *                  y rounded to nearest even; int32 output is acc itself.
 *   Divisions are correctly rounded; bf16 inputs widen exactly to fp32.
 *
 * Packed bit planes (the only persistent format):
 *   Kp = round_up(K, 64), row_bytes = Kp / 8.  A plane is row-major, one row of
 *   row_bytes bytes per matrix row; byte b, bit j (LSB = 0) holds k = 8b + j,
 *   and bits k >= K are 0.  Little-endian 32/64-bit views of the same bytes hold
 *   k = 32w + j / 64w + j.
 *   Binary matrix: one "sign" plane, bit = 1 where the value is -1.
 *   Ternary matrix: a "mask" plane (bit = 1 where t != 0) and a "sign" plane
 *   (bit = 1 where t = -1); sign is a subset of mask.
 *
 * Memory and streams:
 *   Every pointer argument except `stream` is device memory owned by the
 *   caller; the library allocates nothing and keeps no per-call state.  Outputs
 *   must not alias inputs.  `stream` is a hipStream_t (NULL = the default
 *   stream); all work is enqueued on it and no call synchronizes.
 *
 * Errors:
 *   Arguments are validated on the host before anything is enqueued:
 *   BWTA_ERR_INVALID for a NULL required pointer, K <= 0, a negative size, a
 *   leading dimension smaller than the row, or an unknown dtype/algo;
 *   BWTA_ERR_ALIGN for a plane pointer that is not 16-byte aligned or a
 *   float/int pointer that is not aligned to its element; BWTA_ERR_UNSUPPORTED
 *   for a valid request outside what this build implements (say M > 16 for
 *   bwta_gemv, or K > BWTA_MAX_K).  A call with zero rows, columns or batch
 *   entries is a no-op that returns BWTA_OK once sizes, dtypes and algo are
 *   checked; its pointers are not examined and may be NULL.  A failed launch
 *   returns BWTA_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *   synchronization.  bwta_last_error() returns a thread-local description of
 *   the last failure.  No C++ exception crosses this interface.
 */
#ifndef BWTA_H_
#define BWTA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BWTA_API_VERSION 2
/* Largest K (reduction length) any call accepts. */
#define BWTA_MAX_K 65536

typedef enum {
  BWTA_OK = 0,
  BWTA_ERR_INVALID = 1,
  BWTA_ERR_ALIGN = 2,
  BWTA_ERR_UNSUPPORTED = 3,
  BWTA_ERR_HIP = 4
} bwta_status;

typedef enum { BWTA_F32 = 0, BWTA_BF16 = 1, BWTA_I32 = 2 } bwta_dtype;

/* Kernel family for the products.  All give the same exact sums.
 *   AUTO      picks the fastest: MFMA, except the popcount GEMV for decode
 *             products of one row, or of two rows whose plane rows are whole
 *             16-byte units.
 *   MFMA      expands the bit planes to FP4 (e2m1) {-1, 0, +1} and multiplies
 *             on the FP4 matrix cores with unit block scales and fp32
 *             accumulation; every partial sum is an integer below 2^24, so the
 *             result is the exact int32 sum.
 *   POPCOUNT  evaluates acc = nnz - 2 * sum_words popcount((w & (mask ^ sign))
 *             | (~w & sign)) on the vector ALUs.
 *   MFMA_I8   expands the planes to int8 {-1, 0, +1} and multiplies on the int8
 *             matrix cores with int32 accumulation.
 * For K <= 64 (one 64-bit word per row) the MFMA families run the popcount
 * kernel.  bwta_gemv with MFMA or MFMA_I8 runs the FP4 decode kernel. */
typedef enum {
  BWTA_ALGO_AUTO = 0,
  BWTA_ALGO_MFMA = 1,
  BWTA_ALGO_POPCOUNT = 2,
  BWTA_ALGO_MFMA_I8 = 3
} bwta_algo;

int bwta_version(void);

/* round_up(K, 64) and round_up(K, 64) / 8; 0 for K <= 0. */
int64_t bwta_padded_k(int64_t K);
int64_t bwta_row_bytes(int64_t K);

/* Binary weights (page: Abstract, binary weights at one bit per value).
 * W: element (r, k) at W[r * stride_row + k * stride_k] (element strides),
 *    dtype BWTA_F32 or BWTA_BF16; rows >= 0, 0 < K <= BWTA_MAX_K.
 *    stride_k = 1 is the row-major fast path; stride_row = 1 with
 *    stride_k = ld packs the columns of a row-major [K, rows] matrix, which is
 *    how V^T is packed per channel for attention.
 * sign: out, rows * row_bytes(K) bytes, 16-byte aligned.
 * alpha: out, rows floats, alpha[r] = tree(|W[r, :]|) / K. */
bwta_status bwta_pack_weights(const void* W, bwta_dtype w_dtype, int64_t rows, int64_t K,
                              int64_t stride_row, int64_t stride_k, uint8_t* sign,
                              float* alpha, void* stream);

/* Two-plane residual binary weights (BiLLM page, Approach: salient weights get a
 * residual, second-order binarization; here every row): plane 1 and alpha1 are
 * bwta_pack_weights' sign plane and scale; plane 2 and alpha2 are the same rule
 * applied to the fp32 residual r = w - alpha1 * s1 (w - alpha1 where w >= 0 or
 * w is -0.0, w + alpha1 where w < 0), so w ~ alpha1 s1 + alpha2 s2.
 * W: rows x K, row r at W + r * stride_row elements (unit stride along k),
 *    BWTA_F32 or BWTA_BF16; rows a multiple of 32 (else BWTA_ERR_UNSUPPORTED).
 * sign: out, 2 * rows * row_bytes(K) bytes, 16-byte aligned; the planes are
 *    interleaved in groups of 32 rows: plane 1 of weight row n is plane row
 *    64 (n / 32) + n % 32, plane 2 is that row + 32.
 * alpha: out, 2 * rows floats in the same interleaved order. */
bwta_status bwta_pack_weights_residual(const void* W, bwta_dtype w_dtype, int64_t rows, int64_t K,
                                       int64_t stride_row, uint8_t* sign, float* alpha,
                                       void* stream);

/* Ternary activations, projected online (page: Abstract, ternary activations
 * with tiny values projected to zero, two bits per value).
 * X: rows x K, row r at X + r * stride_row elements, unit stride along k,
 *    dtype BWTA_F32 or BWTA_BF16.
 * mask, sign: out, rows * row_bytes(K) bytes each, 16-byte aligned.
 * alpha: out, rows floats; nnz: out, rows int32. */
bwta_status bwta_ternarize_pack(const void* X, bwta_dtype x_dtype, int64_t rows, int64_t K,
                                int64_t stride_row, uint8_t* mask, uint8_t* sign, float* alpha,
                                int32_t* nnz, void* stream);

/* Workspace (bwta_gemm, bwta_gemv).  A product may split its K range across
 * thread blocks; each block then stores an exact int32 partial of its outputs
 * in the workspace (device-coherent stores) and counts itself in a per-tile
 * arrival counter there, and the last block of a tile adds the partials,
 * applies the epilogue and sets the counter back to zero.  The decode kernel does so where it would otherwise
 * split K inside a block (fewer than 1536 tiles of 16 weight rows, LLaMA2-70B
 * down for example).
 *   workspace = NULL: no cross-block split (ws_bytes is ignored); the result is
 *     the same, bit for bit.
 *   Otherwise: device memory owned by the caller, 256-byte aligned
 *     (BWTA_ERR_ALIGN), at least the size query's bytes for the call's shape
 *     and algo (BWTA_ERR_INVALID if smaller; a size of 0 means the call does
 *     not use it).  It must be zero-filled once before its first use; every
 *     call that completes leaves its counters zero again, so the same buffer
 *     serves any later call of any shape.  Calls that share a workspace must
 *     not run concurrently (calls on one stream never do). */
size_t bwta_gemm_workspace_size(int64_t M, int64_t N, int64_t K, bwta_algo algo);
size_t bwta_gemv_workspace_size(int64_t M, int64_t N, int64_t K, bwta_algo algo);

/* Prefill linear (page: Abstract, binary/ternary MatMul for linear operators):
 * Y[m][n] = epilogue(sum_k t[m][k] * s[n][k]) for a ternary A [M x K] (a_mask,
 * a_sign, a_alpha, a_nnz as written by bwta_ternarize_pack) and a binary
 * W [N x K] (w_sign, w_alpha as written by bwta_pack_weights).
 * Y: M x N, row-major with leading dimension ldy >= N (elements), dtype
 *    BWTA_F32, BWTA_BF16 or BWTA_I32 (raw accumulators; a_alpha and w_alpha
 *    may then be NULL).
 * With BWTA_ALGO_AUTO a product of M <= 16 rows runs on the decode kernels of
 * bwta_gemv.  workspace, ws_bytes: see "Workspace" above (NULL allowed). */
bwta_status bwta_gemm(const uint8_t* a_mask, const uint8_t* a_sign, const float* a_alpha,
                      const int32_t* a_nnz, const uint8_t* w_sign, const float* w_alpha,
                      int64_t M, int64_t N, int64_t K, void* Y, bwta_dtype y_dtype, int64_t ldy,
                      bwta_algo algo, void* workspace, size_t ws_bytes, void* stream);

/* Prefill linear with two-plane residual weights (w_sign, w_alpha as written by
 * bwta_pack_weights_residual for N weight rows, 2N plane rows):
 *   Y[m][n] = fl32(fl32(acc1 * fl32(alpha_a[m] * alpha1[n]))
 *               + fl32(acc2 * fl32(alpha_a[m] * alpha2[n])))
 * with acc_i = sum_k t[m][k] * s_i[n][k], both planes multiplied in one pass on
 * the FP4 matrix cores (K <= 64, plane rows of one word: a popcount kernel).
 * Y: M x N, leading dimension ldy >= N, BWTA_F32 or BWTA_BF16.  N must be a
 * multiple of 32 (else BWTA_ERR_UNSUPPORTED); a_nnz is not used and may be
 * NULL. */
bwta_status bwta_gemm_residual(const uint8_t* a_mask, const uint8_t* a_sign, const float* a_alpha,
                               const int32_t* a_nnz, const uint8_t* w_sign, const float* w_alpha,
                               int64_t M, int64_t N, int64_t K, void* Y, bwta_dtype y_dtype,
                               int64_t ldy, void* stream);

/* Decode with two-plane residual weights, 1 <= M <= 16: the product of
 * bwta_gemm_residual by kernels that stream both planes from HBM once (M = 1
 * with row_bytes(K) a multiple of 16: a popcount kernel that reads the four
 * plane rows of two adjacent outputs per wave; otherwise the FP4 decode kernel
 * with each wave on both plane tiles of its 16 outputs).  Any K > 0; N a
 * multiple of 32 and M <= 16 (else BWTA_ERR_UNSUPPORTED); a_nnz is required. */
bwta_status bwta_gemv_residual(const uint8_t* a_mask, const uint8_t* a_sign, const float* a_alpha,
                               const int32_t* a_nnz, const uint8_t* w_sign, const float* w_alpha,
                               int64_t M, int64_t N, int64_t K, void* Y, bwta_dtype y_dtype,
                               int64_t ldy, void* stream);

/* Decode GEMV / skinny GEMM, 1 <= M <= 16: the same product as bwta_gemm with
 * kernels that stream the packed weights from HBM once (page: Abstract, lower
 * memory footprint; the replies quoted on the page name prefill and decode as
 * the workloads).  M > 16 returns BWTA_ERR_UNSUPPORTED.  workspace, ws_bytes:
 * see "Workspace" above (NULL allowed). */
bwta_status bwta_gemv(const uint8_t* a_mask, const uint8_t* a_sign, const float* a_alpha,
                      const int32_t* a_nnz, const uint8_t* w_sign, const float* w_alpha,
                      int64_t M, int64_t N, int64_t K, void* Y, bwta_dtype y_dtype, int64_t ldy,
                      bwta_algo algo, void* workspace, size_t ws_bytes, void* stream);

/* Decode linear in one launch (page: Abstract, ternary activations projected
 * online and a bit-packed binary/ternary MatMul; the replies quoted on the page
 * name decode as a workload): ternarize the M rows of X by the rule of
 * bwta_ternarize_pack and multiply them with the binary weights as bwta_gemv
 * does.  How the rows are ternarized depends on the workspace:
 *   at least bwta_gemv_fused_workspace_size(M, N, K) bytes: each row once, by
 *     one thread block, into exchange buffers (a_mask ... a_nnz when given,
 *     else workspace memory) that the other blocks wait for (a bounded wait:
 *     a block that waits too long ternarizes the rows itself) and then stage
 *     as bwta_gemv does;
 *   otherwise (NULL or smaller): every thread block ternarizes the rows
 *     itself (M * K values per block) and the planes never go through memory.
 * One row that fits the popcount decode kernel (below) always takes the
 * second form, which is the faster one there.
 * X: M x K, row m at X + m * ldx elements, unit stride along k, BWTA_F32 or
 *    BWTA_BF16; 0 <= M <= 16 (else BWTA_ERR_UNSUPPORTED).
 * w_sign, w_alpha, Y, y_dtype, ldy: as for bwta_gemv.  One row (M = 1, K a
 *    multiple of 8 up to 32768 (bf16) or 16384 (fp32), row_bytes(K) a multiple
 *    of 16, X 16-byte aligned) runs on the popcount decode kernel; everything
 *    else on the FP4 decode kernel.  The results are the same either way.
 * a_mask, a_sign (M * row_bytes(K) bytes each, 16-byte aligned) and a_alpha,
 *    a_nnz (M entries): optional outputs, the ternarized planes and scales as
 *    bwta_ternarize_pack would write them; NULL (each pair together) = not
 *    written.
 * workspace, ws_bytes: as for bwta_gemv (NULL allowed; if given, at least
 *    bwta_gemv_workspace_size(M, N, K, BWTA_ALGO_MFMA) bytes, zero-filled once
 *    before its first use; every call leaves it as the next call needs it). */
bwta_status bwta_gemv_fused(const void* X, bwta_dtype x_dtype, int64_t ldx, const uint8_t* w_sign,
                            const float* w_alpha, int64_t M, int64_t N, int64_t K, void* Y,
                            bwta_dtype y_dtype, int64_t ldy, uint8_t* a_mask, uint8_t* a_sign,
                            float* a_alpha, int32_t* a_nnz, void* workspace, size_t ws_bytes,
                            void* stream);

/* Workspace bytes with which bwta_gemv_fused ternarizes each row once: the
 * decode kernel's own workspace, 256 bytes of row flags and room for the
 * exchange planes and scales.  0 for M < 1, M > 16, N < 1 or K out of range. */
size_t bwta_gemv_fused_workspace_size(int64_t M, int64_t N, int64_t K);

/* Test hook of bwta_gemv_fused's bounded wait: the number of polls of the row
 * flags after which a thread block ternarizes the rows itself (default 65536;
 * a negative value restores it).  0 makes every block ternarize every row, the
 * path a block takes if the blocks that own the rows have not run in time.
 * The result is the same either way.  Affects calls made after it returns. */
void bwta_set_fused_spin_limit(int32_t polls);

/* bwta_gemv for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and result as bwta_gemv without the workspace: where bwta_gemv
 * would use a workspace, this call uses the library's own scratch array, a
 * file-scope device array of 4 MiB + 8 KiB of which every GPU the library runs
 * on holds one copy until the process ends.  It allocates nothing (no hipMalloc,
 * hipFree or allocating library call).  Shapes whose workspace would exceed the
 * array return BWTA_ERR_UNSUPPORTED (no decode shape does: every split plan is
 * capped at 4 MiB of partials).  The first call on a device looks up that
 * device's copy and clears its counters with a small kernel on `stream`; every
 * call leaves them zero.  All calls on one GPU share the array: calls that
 * overlap in time on one GPU (different streams, different threads) race and
 * may give wrong results; calls on one stream are ordered and safe. */
bwta_status bwta_gemv_noalloc(const uint8_t* a_mask, const uint8_t* a_sign, const float* a_alpha,
                              const int32_t* a_nnz, const uint8_t* w_sign, const float* w_alpha,
                              int64_t M, int64_t N, int64_t K, void* Y, bwta_dtype y_dtype,
                              int64_t ldy, bwta_algo algo, void* stream);

/* Batched products for attention (page: Abstract, binary/ternary MatMul for
 * attention operators).  For b in [0, batch):
 *   A_b = rows [b * a_batch_rows, b * a_batch_rows + M) of the ternary planes
 *         a_mask/a_sign (and of a_alpha, a_nnz);
 *   B_b = rows [b * b_batch_rows, b * b_batch_rows + N) of B; B is ternary
 *         (b_mask, b_sign) when b_mask != NULL - ternary x ternary, as in
 *         Q K^T - and binary (b_sign only) when b_mask == NULL - as in P V with
 *         V^T packed per channel;
 *   Y_b = Y + b * y_batch_stride elements, M x N with leading dimension ldy.
 * The epilogue scales by a_alpha[row] * b_alpha[col] unless y_dtype is
 * BWTA_I32 (raw scores). */
bwta_status bwta_batched_gemm(int64_t batch, const uint8_t* a_mask, const uint8_t* a_sign,
                              const float* a_alpha, const int32_t* a_nnz, int64_t a_batch_rows,
                              const uint8_t* b_mask, const uint8_t* b_sign, const float* b_alpha,
                              int64_t b_batch_rows, int64_t M, int64_t N, int64_t K, void* Y,
                              bwta_dtype y_dtype, int64_t ldy, int64_t y_batch_stride,
                              bwta_algo algo, void* stream);

/* Fused attention (page: Abstract and "Core claim", binary/ternary MatMul for
 * the attention operators).  For every head h < heads and query row i < L, in
 * one launch:
 *   S[j]  = sum_d t_q[i, d] t_k[j, d] over d < D      (ternary x ternary)
 *   P[j]  = softmax over j < L of alpha_q[i] alpha_k[j] S[j] * scale, in fp32:
 *           u = S * alpha_k[j]; a = alpha_q[i] * scale * log2(e);
 *           e_j = exp2(fma(a, u_j, -(a * max u))); p_j = e_j * (1 / sum e)
 *   t_p, alpha_p, nnz_p = ternarize(P row) by the rule of bwta_ternarize_pack
 *           (tree(|p|) / L, threshold 0.5 * mu, alpha over the kept values)
 *   O[i, c] = fl32((nnz_p - 2 sum_j t_p[j] b_v[c, j]) * fl32(alpha_p * alpha_v[c]))
 *           for every channel c < D, with b_v the V^T sign bits (1 = negative).
 * The scores and P stay on chip; only O is written unless the optional
 * outputs are given.
 * q_mask, q_sign, k_mask, k_sign: heads * L rows of row_bytes(D) bytes (as
 *    written by bwta_ternarize_pack for [heads * L, D] inputs), 16-byte aligned;
 *    q_alpha, k_alpha: heads * L floats, 16-byte aligned (nnz is not needed).
 * v_sign: V^T planes, heads * D rows (row h * D + c = channel c of head h) of
 *    row_bytes(L) bytes, as written by bwta_pack_weights with stride_row = 1
 *    over a [L, heads * D] V; v_alpha: heads * D floats; both 16-byte aligned.
 * O: [heads * L, D] row-major, BWTA_F32 or BWTA_BF16, 16-byte aligned.
 * Optional (NULL: not written), for inspection: p_out [heads * L, L] fp32 (P),
 *    p_mask [heads * L, row_bytes(L)] (t_p; its sign plane is all zero since
 *    every p >= 0), p_alpha [heads * L] floats, p_nnz [heads * L] int32;
 *    16-byte aligned (p_alpha, p_nnz: 4-byte).
 * Supported shapes: D = 128 and L in {512, 1024, 2048}, heads <= 65535; other
 * shapes return BWTA_ERR_UNSUPPORTED.  heads = 0 is a no-op. */
bwta_status bwta_attention(int64_t heads, int64_t L, int64_t D, const uint8_t* q_mask,
                           const uint8_t* q_sign, const float* q_alpha, const uint8_t* k_mask,
                           const uint8_t* k_sign, const float* k_alpha, const uint8_t* v_sign,
                           const float* v_alpha, float scale, void* O, bwta_dtype o_dtype,
                           float* p_out, uint8_t* p_mask, float* p_alpha, int32_t* p_nnz,
                           void* stream);

const char* bwta_status_string(bwta_status status);
const char* bwta_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BWTA_H_ */
