// bwta_api.cpp - the extern "C" entry points of libbwta.so: argument
// validation, status codes, kernel selection.  Definitions of the operations
// are in bwta.h; the kernels are in pack.hip, gemm_mfma.hip, gemm_mfma_i8.hip,
// gemm_popcount.hip, gemv_mfma.hip and attention.hip.
#include "bwta.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kernels.hpp"

namespace {

thread_local char g_last_error[512] = "";

// Polls of the row flags before a block of the ternarize-once decode
// ternarizes the rows itself (bwta_set_fused_spin_limit).
constexpr int kDefaultFusedSpin = 1 << 16;
std::atomic<int> g_fused_spin{kDefaultFusedSpin};

bwta_status fail(bwta_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

bwta_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return BWTA_OK;
  return fail(BWTA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_io_dtype(bwta_dtype d) { return d == BWTA_F32 || d == BWTA_BF16; }
bool valid_out_dtype(bwta_dtype d) { return d == BWTA_F32 || d == BWTA_BF16 || d == BWTA_I32; }
size_t dtype_size(bwta_dtype d) { return d == BWTA_BF16 ? 2 : 4; }

bwta_status check_plane(const void* p, const char* name) {
  if (!p) return fail(BWTA_ERR_INVALID, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(BWTA_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return BWTA_OK;
}

bwta_status check_word(const void* p, bool required, const char* name) {
  if (!p) return required ? fail(BWTA_ERR_INVALID, "%s is NULL", name) : BWTA_OK;
  if (!aligned(p, 4)) return fail(BWTA_ERR_ALIGN, "%s is not 4-byte aligned", name);
  return BWTA_OK;
}

bwta_status check_k(int64_t K) {
  if (K <= 0) return fail(BWTA_ERR_INVALID, "K must be positive (got %lld)", (long long)K);
  if (K > BWTA_MAX_K)
    return fail(BWTA_ERR_UNSUPPORTED, "K = %lld exceeds BWTA_MAX_K = %d", (long long)K, BWTA_MAX_K);
  return BWTA_OK;
}

#define BWTA_TRY(x)                  \
  do {                               \
    bwta_status st_ = (x);           \
    if (st_ != BWTA_OK) return st_;  \
  } while (0)

bwta_status check_product(const uint8_t* a_mask, const uint8_t* a_sign, const float* a_alpha,
                          const int32_t* a_nnz, const uint8_t* b_mask, bool b_ternary,
                          const uint8_t* b_sign, const float* b_alpha, int64_t M, int64_t N,
                          int64_t K, const void* Y, bwta_dtype y_dtype, int64_t ldy,
                          bwta_algo algo) {
  if (M < 0 || N < 0) return fail(BWTA_ERR_INVALID, "negative size M=%lld N=%lld", (long long)M, (long long)N);
  BWTA_TRY(check_k(K));
  if (!valid_out_dtype(y_dtype)) return fail(BWTA_ERR_INVALID, "bad output dtype %d", (int)y_dtype);
  if (algo != BWTA_ALGO_AUTO && algo != BWTA_ALGO_MFMA && algo != BWTA_ALGO_POPCOUNT &&
      algo != BWTA_ALGO_MFMA_I8)
    return fail(BWTA_ERR_INVALID, "bad algo %d", (int)algo);
  if (ldy < N) return fail(BWTA_ERR_INVALID, "ldy (%lld) < N (%lld)", (long long)ldy, (long long)N);
  if (M == 0 || N == 0) return BWTA_OK;  // empty: pointers may be NULL
  BWTA_TRY(check_plane(a_mask, "a_mask"));
  BWTA_TRY(check_plane(a_sign, "a_sign"));
  if (b_ternary) BWTA_TRY(check_plane(b_mask, "b_mask"));
  BWTA_TRY(check_plane(b_sign, b_ternary ? "b_sign" : "w_sign"));
  const bool scaled = y_dtype != BWTA_I32;
  BWTA_TRY(check_word(a_alpha, scaled, "a_alpha"));
  BWTA_TRY(check_word(b_alpha, scaled, b_ternary ? "b_alpha" : "w_alpha"));
  BWTA_TRY(check_word(a_nnz, !b_ternary, "a_nnz"));
  if (!Y) return fail(BWTA_ERR_INVALID, "Y is NULL");
  if (!aligned(Y, dtype_size(y_dtype))) return fail(BWTA_ERR_ALIGN, "Y is not aligned to its element");
  return BWTA_OK;
}

// AUTO on a decode product (binary B): one activation row, or two whose plane
// rows are whole 16-byte units, cost the popcount GEMV one merge and one
// population count per weight word and row, less than building FP4 operands
// (LLaMA2-70B gate/up and down at M = 2: 8.25 and 8.37 us against 8.43 and
// 8.97 us); from three rows on the FP4 GEMV, whose cost does not grow with M,
// is faster (M = 3: 17.8 against 8.4 us).
bool auto_popcount_decode(int64_t M, int64_t K) {
  return M <= 1 || (M == 2 && ((K + 63) / 64 * 8) % 16 == 0);
}

// Workspace bytes of one product call: the decode kernel's cross-block K split
// is the only user.  gemv: the FP4 decode kernel (AUTO where the popcount GEMV
// does not take the rows, MFMA, MFMA_I8); gemm: AUTO sends M <= 16 to the same
// decode kernels.
size_t product_workspace(int64_t M, int64_t N, int64_t K, bwta_algo algo, bool gemv) {
  if (M <= 0 || N <= 0 || K <= 0 || K > BWTA_MAX_K || M > 16) return 0;
  bool fp4_decode;
  if (gemv)
    fp4_decode = algo == BWTA_ALGO_MFMA || algo == BWTA_ALGO_MFMA_I8 ||
                 (algo == BWTA_ALGO_AUTO && !auto_popcount_decode(M, K));
  else
    fp4_decode = algo == BWTA_ALGO_AUTO && !auto_popcount_decode(M, K);
  return fp4_decode ? bwta::gemv_mfma_workspace_bytes(M, N, K) : 0;
}

bwta_status check_workspace(const void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return BWTA_OK;  // no workspace: no cross-block split
  if (!aligned(ws, 256)) return fail(BWTA_ERR_ALIGN, "workspace is not 256-byte aligned");
  if (ws_bytes < need)
    return fail(BWTA_ERR_INVALID, "workspace of %zu bytes is smaller than the %zu this call needs",
                ws_bytes, need);
  return BWTA_OK;
}

bwta::Elt elt(bwta_dtype d) {
  return d == BWTA_F32 ? bwta::Elt::F32 : d == BWTA_BF16 ? bwta::Elt::BF16 : bwta::Elt::I32;
}

}  // namespace

extern "C" {

int bwta_version(void) { return BWTA_API_VERSION; }

int64_t bwta_padded_k(int64_t K) { return K <= 0 ? 0 : (K + 63) / 64 * 64; }
int64_t bwta_row_bytes(int64_t K) { return bwta_padded_k(K) / 8; }

const char* bwta_status_string(bwta_status s) {
  switch (s) {
    case BWTA_OK: return "BWTA_OK";
    case BWTA_ERR_INVALID: return "BWTA_ERR_INVALID";
    case BWTA_ERR_ALIGN: return "BWTA_ERR_ALIGN";
    case BWTA_ERR_UNSUPPORTED: return "BWTA_ERR_UNSUPPORTED";
    case BWTA_ERR_HIP: return "BWTA_ERR_HIP";
  }
  return "BWTA_ERR_UNKNOWN";
}

const char* bwta_last_error(void) { return g_last_error; }

bwta_status bwta_pack_weights(const void* W, bwta_dtype w_dtype, int64_t rows, int64_t K,
                              int64_t stride_row, int64_t stride_k, uint8_t* sign, float* alpha,
                              void* stream) {
  if (!valid_io_dtype(w_dtype)) return fail(BWTA_ERR_INVALID, "bad weight dtype %d", (int)w_dtype);
  if (rows < 0) return fail(BWTA_ERR_INVALID, "negative rows");
  BWTA_TRY(check_k(K));
  if (stride_row < 0 || stride_k <= 0) return fail(BWTA_ERR_INVALID, "bad strides");
  if (rows == 0) return BWTA_OK;  // empty: pointers may be NULL
  if (!W) return fail(BWTA_ERR_INVALID, "W is NULL");
  if (!aligned(W, dtype_size(w_dtype))) return fail(BWTA_ERR_ALIGN, "W is not aligned to its element");
  BWTA_TRY(check_plane(sign, "sign"));
  BWTA_TRY(check_word(alpha, true, "alpha"));
  if (rows == 0) return BWTA_OK;
  return from_hip(bwta::launch_binarize(W, elt(w_dtype), rows, K, stride_row, stride_k, sign, alpha,
                                        static_cast<hipStream_t>(stream)),
                  "bwta_pack_weights launch");
}

bwta_status bwta_pack_weights_residual(const void* W, bwta_dtype w_dtype, int64_t rows, int64_t K,
                                       int64_t stride_row, uint8_t* sign, float* alpha,
                                       void* stream) {
  if (!valid_io_dtype(w_dtype)) return fail(BWTA_ERR_INVALID, "bad weight dtype %d", (int)w_dtype);
  if (rows < 0) return fail(BWTA_ERR_INVALID, "negative rows");
  BWTA_TRY(check_k(K));
  if (stride_row < K && rows > 1) return fail(BWTA_ERR_INVALID, "stride_row < K");
  if (rows % 32 != 0)
    return fail(BWTA_ERR_UNSUPPORTED, "rows = %lld is not a multiple of 32", (long long)rows);
  if (rows == 0) return BWTA_OK;  // empty: pointers may be NULL
  if (!W) return fail(BWTA_ERR_INVALID, "W is NULL");
  if (!aligned(W, dtype_size(w_dtype))) return fail(BWTA_ERR_ALIGN, "W is not aligned to its element");
  BWTA_TRY(check_plane(sign, "sign"));
  BWTA_TRY(check_word(alpha, true, "alpha"));
  return from_hip(bwta::launch_binarize_residual(W, elt(w_dtype), rows, K, stride_row, sign, alpha,
                                                 static_cast<hipStream_t>(stream)),
                  "bwta_pack_weights_residual launch");
}

bwta_status bwta_ternarize_pack(const void* X, bwta_dtype x_dtype, int64_t rows, int64_t K,
                                int64_t stride_row, uint8_t* mask, uint8_t* sign, float* alpha,
                                int32_t* nnz, void* stream) {
  if (!valid_io_dtype(x_dtype)) return fail(BWTA_ERR_INVALID, "bad activation dtype %d", (int)x_dtype);
  if (rows < 0) return fail(BWTA_ERR_INVALID, "negative rows");
  BWTA_TRY(check_k(K));
  if (stride_row < K && rows > 1) return fail(BWTA_ERR_INVALID, "stride_row < K");
  if (rows == 0) return BWTA_OK;  // empty: pointers may be NULL
  if (!X) return fail(BWTA_ERR_INVALID, "X is NULL");
  if (!aligned(X, dtype_size(x_dtype))) return fail(BWTA_ERR_ALIGN, "X is not aligned to its element");
  BWTA_TRY(check_plane(mask, "mask"));
  BWTA_TRY(check_plane(sign, "sign"));
  BWTA_TRY(check_word(alpha, true, "alpha"));
  BWTA_TRY(check_word(nnz, true, "nnz"));
  if (rows == 0) return BWTA_OK;
  return from_hip(bwta::launch_ternarize(X, elt(x_dtype), rows, K, stride_row, mask, sign, alpha,
                                         nnz, static_cast<hipStream_t>(stream)),
                  "bwta_ternarize_pack launch");
}

static bwta_status run_product(const bwta::GemmArgs& g, bwta_algo algo, bool gemv,
                               hipStream_t stream) {
  const int64_t row_bytes = (g.K + 63) / 64 * 8;
  // A single (unbatched) product of at most 16 activation rows is a decode
  // product: with AUTO, bwta_gemm runs it on the decode kernels as well.
  if (!gemv && algo == BWTA_ALGO_AUTO && g.batch == 1 && !g.b_mask && g.M <= 16) gemv = true;
  if (algo == BWTA_ALGO_AUTO)
    algo = (gemv && !g.b_mask && auto_popcount_decode(g.M, g.K)) ? BWTA_ALGO_POPCOUNT
                                                                 : BWTA_ALGO_MFMA;
  hipError_t e;
  if (gemv && !g.b_mask && (algo == BWTA_ALGO_MFMA || algo == BWTA_ALGO_MFMA_I8)) {
    // Decode: the skinny FP4 kernel streams the weights once for any M <= 16.
    e = bwta::launch_gemv_mfma(g, stream);
    return from_hip(e, "gemv launch");
  }
  if (algo == BWTA_ALGO_POPCOUNT) {
    if (gemv && !g.b_mask && row_bytes % 16 == 0)
      e = bwta::launch_gemv_popcount(g, stream);
    else
      e = bwta::launch_gemm_popcount(g, stream);
  } else if (g.K <= 64) {
    // One 64-bit word per row: below the MFMA kernel's 16-byte DMA window;
    // the popcount kernel computes the same exact sums.
    e = bwta::launch_gemm_popcount(g, stream);
  } else if (algo == BWTA_ALGO_MFMA_I8) {
    e = bwta::launch_gemm_mfma_i8(g, stream);
  } else {
    e = bwta::launch_gemm_mfma(g, stream);
  }
  return from_hip(e, "product launch");
}

size_t bwta_gemm_workspace_size(int64_t M, int64_t N, int64_t K, bwta_algo algo) {
  return product_workspace(M, N, K, algo, false);
}

size_t bwta_gemv_workspace_size(int64_t M, int64_t N, int64_t K, bwta_algo algo) {
  return product_workspace(M, N, K, algo, true);
}

bwta_status bwta_gemm(const uint8_t* a_mask, const uint8_t* a_sign, const float* a_alpha,
                      const int32_t* a_nnz, const uint8_t* w_sign, const float* w_alpha, int64_t M,
                      int64_t N, int64_t K, void* Y, bwta_dtype y_dtype, int64_t ldy,
                      bwta_algo algo, void* workspace, size_t ws_bytes, void* stream) {
  BWTA_TRY(check_product(a_mask, a_sign, a_alpha, a_nnz, nullptr, false, w_sign, w_alpha, M, N, K,
                         Y, y_dtype, ldy, algo));
  if (M == 0 || N == 0) return BWTA_OK;
  const size_t need = product_workspace(M, N, K, algo, false);
  BWTA_TRY(check_workspace(workspace, ws_bytes, need));
  bwta::GemmArgs g{a_mask, a_sign, a_alpha, a_nnz, 0, nullptr, w_sign, w_alpha, 0,
                   1, M, N, K, Y, elt(y_dtype), ldy, 0};
  if (need > 0) {
    g.ws = workspace;
    g.ws_bytes = ws_bytes;
  }
  return run_product(g, algo, false, static_cast<hipStream_t>(stream));
}

bwta_status bwta_gemm_residual(const uint8_t* a_mask, const uint8_t* a_sign, const float* a_alpha,
                               const int32_t* a_nnz, const uint8_t* w_sign, const float* w_alpha,
                               int64_t M, int64_t N, int64_t K, void* Y, bwta_dtype y_dtype,
                               int64_t ldy, void* stream) {
  (void)a_nnz;  // the two-plane product does not use nnz
  if (M < 0 || N < 0) return fail(BWTA_ERR_INVALID, "negative size M=%lld N=%lld", (long long)M, (long long)N);
  BWTA_TRY(check_k(K));
  if (!valid_io_dtype(y_dtype)) return fail(BWTA_ERR_INVALID, "bad output dtype %d", (int)y_dtype);
  if (ldy < N) return fail(BWTA_ERR_INVALID, "ldy (%lld) < N (%lld)", (long long)ldy, (long long)N);
  if (N % 32 != 0)
    return fail(BWTA_ERR_UNSUPPORTED, "N = %lld is not a multiple of 32", (long long)N);
  if (M == 0 || N == 0) return BWTA_OK;  // empty: pointers may be NULL
  BWTA_TRY(check_plane(a_mask, "a_mask"));
  BWTA_TRY(check_plane(a_sign, "a_sign"));
  BWTA_TRY(check_plane(w_sign, "w_sign"));
  BWTA_TRY(check_word(a_alpha, true, "a_alpha"));
  BWTA_TRY(check_word(w_alpha, true, "w_alpha"));
  if (!Y) return fail(BWTA_ERR_INVALID, "Y is NULL");
  if (!aligned(Y, dtype_size(y_dtype))) return fail(BWTA_ERR_ALIGN, "Y is not aligned to its element");
  bwta::GemmArgs g{a_mask, a_sign, a_alpha, a_nnz, 0, nullptr, w_sign, w_alpha, 0,
                   1, M, 2 * N, K, Y, elt(y_dtype), ldy, 0};
  // The FP4 kernel's 16-byte DMA window needs plane rows of 16 bytes or more
  // (K > 64); rows of one word take the popcount kernel.
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(K <= 64 ? bwta::launch_gemm_residual_word(g, st)
                          : bwta::launch_gemm_mfma_residual(g, st),
                  "bwta_gemm_residual launch");
}

bwta_status bwta_gemv_residual(const uint8_t* a_mask, const uint8_t* a_sign, const float* a_alpha,
                               const int32_t* a_nnz, const uint8_t* w_sign, const float* w_alpha,
                               int64_t M, int64_t N, int64_t K, void* Y, bwta_dtype y_dtype,
                               int64_t ldy, void* stream) {
  if (M < 0 || N < 0) return fail(BWTA_ERR_INVALID, "negative size M=%lld N=%lld", (long long)M, (long long)N);
  BWTA_TRY(check_k(K));
  if (!valid_io_dtype(y_dtype)) return fail(BWTA_ERR_INVALID, "bad output dtype %d", (int)y_dtype);
  if (ldy < N) return fail(BWTA_ERR_INVALID, "ldy (%lld) < N (%lld)", (long long)ldy, (long long)N);
  if (M > 16) return fail(BWTA_ERR_UNSUPPORTED, "bwta_gemv_residual takes M <= 16 (got %lld)", (long long)M);
  if (N % 32 != 0)
    return fail(BWTA_ERR_UNSUPPORTED, "N = %lld is not a multiple of 32", (long long)N);
  if (M == 0 || N == 0) return BWTA_OK;  // empty: pointers may be NULL
  BWTA_TRY(check_plane(a_mask, "a_mask"));
  BWTA_TRY(check_plane(a_sign, "a_sign"));
  BWTA_TRY(check_plane(w_sign, "w_sign"));
  BWTA_TRY(check_word(a_alpha, true, "a_alpha"));
  BWTA_TRY(check_word(a_nnz, true, "a_nnz"));
  BWTA_TRY(check_word(w_alpha, true, "w_alpha"));
  if (!Y) return fail(BWTA_ERR_INVALID, "Y is NULL");
  if (!aligned(Y, dtype_size(y_dtype))) return fail(BWTA_ERR_ALIGN, "Y is not aligned to its element");
  // One activation row: the popcount GEMV (16-byte words of each plane row;
  // 70B gate/up 11.4 us, 5.2 TB/s); more rows or other row lengths: the FP4
  // GEMV, whose cost does not grow with M.
  const int64_t row_bytes = (K + 63) / 64 * 8;
  bwta::GemmArgs g{a_mask, a_sign, a_alpha, a_nnz, 0, nullptr, w_sign, w_alpha, 0,
                   1, M, N, K, Y, elt(y_dtype), ldy, 0};
  const hipError_t e = row_bytes % 16 == 0 && M == 1
                           ? bwta::launch_gemv_popcount_residual(g, static_cast<hipStream_t>(stream))
                           : bwta::launch_gemv_mfma_residual(g, static_cast<hipStream_t>(stream));
  return from_hip(e, "bwta_gemv_residual launch");
}

bwta_status bwta_gemv(const uint8_t* a_mask, const uint8_t* a_sign, const float* a_alpha,
                      const int32_t* a_nnz, const uint8_t* w_sign, const float* w_alpha, int64_t M,
                      int64_t N, int64_t K, void* Y, bwta_dtype y_dtype, int64_t ldy,
                      bwta_algo algo, void* workspace, size_t ws_bytes, void* stream) {
  BWTA_TRY(check_product(a_mask, a_sign, a_alpha, a_nnz, nullptr, false, w_sign, w_alpha, M, N, K,
                         Y, y_dtype, ldy, algo));
  if (M > 16) return fail(BWTA_ERR_UNSUPPORTED, "bwta_gemv takes M <= 16 (got %lld)", (long long)M);
  if (M == 0 || N == 0) return BWTA_OK;
  const size_t need = product_workspace(M, N, K, algo, true);
  BWTA_TRY(check_workspace(workspace, ws_bytes, need));
  bwta::GemmArgs g{a_mask, a_sign, a_alpha, a_nnz, 0, nullptr, w_sign, w_alpha, 0,
                   1, M, N, K, Y, elt(y_dtype), ldy, 0};
  if (need > 0) {
    g.ws = workspace;
    g.ws_bytes = ws_bytes;
  }
  return run_product(g, algo, true, static_cast<hipStream_t>(stream));
}

bwta_status bwta_gemv_fused(const void* X, bwta_dtype x_dtype, int64_t ldx, const uint8_t* w_sign,
                            const float* w_alpha, int64_t M, int64_t N, int64_t K, void* Y,
                            bwta_dtype y_dtype, int64_t ldy, uint8_t* a_mask, uint8_t* a_sign,
                            float* a_alpha, int32_t* a_nnz, void* workspace, size_t ws_bytes,
                            void* stream) {
  if (!valid_io_dtype(x_dtype)) return fail(BWTA_ERR_INVALID, "bad activation dtype %d", (int)x_dtype);
  if (M < 0 || N < 0) return fail(BWTA_ERR_INVALID, "negative size M=%lld N=%lld", (long long)M, (long long)N);
  BWTA_TRY(check_k(K));
  if (!valid_out_dtype(y_dtype)) return fail(BWTA_ERR_INVALID, "bad output dtype %d", (int)y_dtype);
  if (ldy < N) return fail(BWTA_ERR_INVALID, "ldy (%lld) < N (%lld)", (long long)ldy, (long long)N);
  if (ldx < K && M > 1) return fail(BWTA_ERR_INVALID, "ldx (%lld) < K (%lld)", (long long)ldx, (long long)K);
  if (M > 16)
    return fail(BWTA_ERR_UNSUPPORTED, "bwta_gemv_fused takes M <= 16 (got %lld)", (long long)M);
  if (N >= ((int64_t)1 << 29)) return fail(BWTA_ERR_UNSUPPORTED, "N >= 2^29");
  if ((a_mask == nullptr) != (a_sign == nullptr))
    return fail(BWTA_ERR_INVALID, "a_mask and a_sign are given together or not at all");
  if ((a_alpha == nullptr) != (a_nnz == nullptr))
    return fail(BWTA_ERR_INVALID, "a_alpha and a_nnz are given together or not at all");
  if (M == 0 || N == 0) return BWTA_OK;  // empty: pointers may be NULL
  if (!X) return fail(BWTA_ERR_INVALID, "X is NULL");
  if (!aligned(X, dtype_size(x_dtype))) return fail(BWTA_ERR_ALIGN, "X is not aligned to its element");
  BWTA_TRY(check_plane(w_sign, "w_sign"));
  BWTA_TRY(check_word(w_alpha, y_dtype != BWTA_I32, "w_alpha"));
  if (!Y) return fail(BWTA_ERR_INVALID, "Y is NULL");
  if (!aligned(Y, dtype_size(y_dtype))) return fail(BWTA_ERR_ALIGN, "Y is not aligned to its element");
  if (a_mask) {
    BWTA_TRY(check_plane(a_mask, "a_mask"));
    BWTA_TRY(check_plane(a_sign, "a_sign"));
  }
  BWTA_TRY(check_word(a_alpha, false, "a_alpha"));
  BWTA_TRY(check_word(a_nnz, false, "a_nnz"));
  const size_t need = bwta::gemv_mfma_workspace_bytes(M, N, K);
  BWTA_TRY(check_workspace(workspace, ws_bytes, need));
  bwta::GemmArgs g{nullptr, nullptr, nullptr, nullptr, 0, nullptr, w_sign, w_alpha, 0,
                   1, M, N, K, Y, elt(y_dtype), ldy, 0};
  if (workspace && need > 0) {
    g.ws = workspace;
    g.ws_bytes = ws_bytes;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // One row: the popcount decode kernel with the ternarization in each block.
  hipError_t e = bwta::launch_gemv_fused_row(g, X, elt(x_dtype), a_mask, a_sign, a_alpha, a_nnz, st);
  if (e != hipErrorNotSupported) return from_hip(e, "bwta_gemv_fused launch");
  // With room for the exchange buffers: each row ternarized once, one launch.
  if (workspace && ws_bytes >= bwta::gemv_fused_xp_workspace_bytes(M, N, K)) {
    e = bwta::launch_gemv_fused_xp(g, X, elt(x_dtype), ldx, a_mask, a_sign, a_alpha, a_nnz,
                                   workspace, ws_bytes, g_fused_spin.load(), st);
    if (e != hipErrorNotSupported) return from_hip(e, "bwta_gemv_fused launch");
  }
  return from_hip(bwta::launch_gemv_fused(g, X, elt(x_dtype), ldx, a_mask, a_sign, a_alpha, a_nnz, st),
                  "bwta_gemv_fused launch");
}

size_t bwta_gemv_fused_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || M > 16 || K > BWTA_MAX_K) return 0;
  const size_t plain = bwta::gemv_mfma_workspace_bytes(M, N, K);
  const size_t xp = bwta::gemv_fused_xp_workspace_bytes(M, N, K);
  return xp > plain ? xp : plain;
}

void bwta_set_fused_spin_limit(int32_t polls) {
  g_fused_spin.store(polls < 0 ? kDefaultFusedSpin : polls);
}

bwta_status bwta_gemv_noalloc(const uint8_t* a_mask, const uint8_t* a_sign, const float* a_alpha,
                              const int32_t* a_nnz, const uint8_t* w_sign, const float* w_alpha,
                              int64_t M, int64_t N, int64_t K, void* Y, bwta_dtype y_dtype,
                              int64_t ldy, bwta_algo algo, void* stream) {
  BWTA_TRY(check_product(a_mask, a_sign, a_alpha, a_nnz, nullptr, false, w_sign, w_alpha, M, N, K,
                         Y, y_dtype, ldy, algo));
  if (M > 16)
    return fail(BWTA_ERR_UNSUPPORTED, "bwta_gemv_noalloc takes M <= 16 (got %lld)", (long long)M);
  if (M == 0 || N == 0) return BWTA_OK;
  const size_t need = product_workspace(M, N, K, algo, true);
  if (need > bwta::scratch_bytes())
    return fail(BWTA_ERR_UNSUPPORTED,
                "this shape needs %zu bytes of workspace, more than the %zu of the library's "
                "scratch array", need, bwta::scratch_bytes());
  bwta::GemmArgs g{a_mask, a_sign, a_alpha, a_nnz, 0, nullptr, w_sign, w_alpha, 0,
                   1, M, N, K, Y, elt(y_dtype), ldy, 0};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (need > 0) {
    void* p = nullptr;
    const hipError_t e = bwta::scratch_workspace(&p, st);
    if (e != hipSuccess) return from_hip(e, "scratch array of bwta_gemv_noalloc");
    g.ws = p;
    g.ws_bytes = bwta::scratch_bytes();
  }
  return run_product(g, algo, true, st);
}

bwta_status bwta_batched_gemm(int64_t batch, const uint8_t* a_mask, const uint8_t* a_sign,
                              const float* a_alpha, const int32_t* a_nnz, int64_t a_batch_rows,
                              const uint8_t* b_mask, const uint8_t* b_sign, const float* b_alpha,
                              int64_t b_batch_rows, int64_t M, int64_t N, int64_t K, void* Y,
                              bwta_dtype y_dtype, int64_t ldy, int64_t y_batch_stride,
                              bwta_algo algo, void* stream) {
  if (batch < 0) return fail(BWTA_ERR_INVALID, "negative batch");
  if (a_batch_rows < 0 || b_batch_rows < 0 || y_batch_stride < 0)
    return fail(BWTA_ERR_INVALID, "negative batch stride");
  if (batch > 65535) return fail(BWTA_ERR_UNSUPPORTED, "batch > 65535");
  if (batch == 0) return BWTA_OK;  // empty: pointers may be NULL
  const bool tern = b_mask != nullptr;
  BWTA_TRY(check_product(a_mask, a_sign, a_alpha, a_nnz, b_mask, tern, b_sign, b_alpha, M, N, K, Y,
                         y_dtype, ldy, algo));
  if (batch == 0 || M == 0 || N == 0) return BWTA_OK;
  bwta::GemmArgs g{a_mask, a_sign, a_alpha, a_nnz, a_batch_rows, b_mask, b_sign, b_alpha,
                   b_batch_rows, batch, M, N, K, Y, elt(y_dtype), ldy, y_batch_stride};
  return run_product(g, algo, false, static_cast<hipStream_t>(stream));
}

bwta_status bwta_attention(int64_t heads, int64_t L, int64_t D, const uint8_t* q_mask,
                           const uint8_t* q_sign, const float* q_alpha, const uint8_t* k_mask,
                           const uint8_t* k_sign, const float* k_alpha, const uint8_t* v_sign,
                           const float* v_alpha, float scale, void* O, bwta_dtype o_dtype,
                           float* p_out, uint8_t* p_mask, float* p_alpha, int32_t* p_nnz,
                           void* stream) {
  if (heads < 0 || L < 0 || D < 0)
    return fail(BWTA_ERR_INVALID, "negative size heads=%lld L=%lld D=%lld", (long long)heads,
                (long long)L, (long long)D);
  if (!valid_io_dtype(o_dtype)) return fail(BWTA_ERR_INVALID, "bad output dtype %d", (int)o_dtype);
  if (!std::isfinite(scale))
    return fail(BWTA_ERR_INVALID, "scale is not finite");
  if (heads == 0) return BWTA_OK;
  if (D != 128) return fail(BWTA_ERR_UNSUPPORTED, "head dim %lld (only 128)", (long long)D);
  if (L != 512 && L != 1024 && L != 2048)
    return fail(BWTA_ERR_UNSUPPORTED, "L = %lld (only 512, 1024, 2048)", (long long)L);
  if (heads > 65535) return fail(BWTA_ERR_UNSUPPORTED, "heads > 65535");
  BWTA_TRY(check_plane(q_mask, "q_mask"));
  BWTA_TRY(check_plane(q_sign, "q_sign"));
  BWTA_TRY(check_plane(q_alpha, "q_alpha"));
  BWTA_TRY(check_plane(k_mask, "k_mask"));
  BWTA_TRY(check_plane(k_sign, "k_sign"));
  BWTA_TRY(check_plane(k_alpha, "k_alpha"));
  BWTA_TRY(check_plane(v_sign, "v_sign"));
  BWTA_TRY(check_plane(v_alpha, "v_alpha"));
  BWTA_TRY(check_plane(O, "O"));
  if (p_out && !aligned(p_out, 16)) return fail(BWTA_ERR_ALIGN, "p_out is not 16-byte aligned");
  if (p_mask && !aligned(p_mask, 16)) return fail(BWTA_ERR_ALIGN, "p_mask is not 16-byte aligned");
  BWTA_TRY(check_word(p_alpha, false, "p_alpha"));
  BWTA_TRY(check_word(p_nnz, false, "p_nnz"));
  bwta::AttentionArgs a{heads, L, D, q_mask, q_sign, q_alpha, k_mask, k_sign, k_alpha, v_sign,
                        v_alpha, scale, O, elt(o_dtype), p_out, p_mask, p_alpha, p_nnz};
  return from_hip(bwta::launch_attention(a, static_cast<hipStream_t>(stream)), "attention launch");
}

}  // extern "C"
