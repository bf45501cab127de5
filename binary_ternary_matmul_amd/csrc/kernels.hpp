// kernels.hpp - host-side launchers of the libbwta kernels (internal).
//
// Arguments reach these functions already validated by bwta_api.cpp; each
// launcher only chooses a kernel configuration and enqueues it on `stream`.
// They return hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bwta {

enum class Elt : int { F32 = 0, BF16 = 1, I32 = 2 };

// Row reduction + bit packing (ternarize_pack and pack_weights).
hipError_t launch_ternarize(const void* X, Elt dt, int64_t rows, int64_t K, int64_t stride_row,
                            uint8_t* mask, uint8_t* sign, float* alpha, int32_t* nnz,
                            hipStream_t stream);
hipError_t launch_binarize(const void* W, Elt dt, int64_t rows, int64_t K, int64_t stride_row,
                           int64_t stride_k, uint8_t* sign, float* alpha, hipStream_t stream);
// Two-plane residual binarization, planes interleaved in groups of 32 rows
// (rows must be a multiple of 32).
hipError_t launch_binarize_residual(const void* W, Elt dt, int64_t rows, int64_t K,
                                   int64_t stride_row, uint8_t* sign, float* alpha,
                                   hipStream_t stream);

// Common description of one (possibly batched) product.
struct GemmArgs {
  const uint8_t* a_mask;
  const uint8_t* a_sign;
  const float* a_alpha;
  const int32_t* a_nnz;
  int64_t a_batch_rows;
  const uint8_t* b_mask;  // nullptr: binary B
  const uint8_t* b_sign;
  const float* b_alpha;
  int64_t b_batch_rows;
  int64_t batch, M, N, K;
  void* Y;
  Elt y_dt;
  int64_t ldy, y_batch_stride;
  // Optional workspace (zero-filled before its first use; every launch leaves
  // its counters zero): enables the decode kernel's cross-block K split.
  void* ws = nullptr;
  size_t ws_bytes = 0;
};

hipError_t launch_gemm_mfma(const GemmArgs& g, hipStream_t stream);
// Two-plane residual weights (B interleaved in groups of 32 rows, g.N = 2 x outputs).
hipError_t launch_gemm_mfma_residual(const GemmArgs& g, hipStream_t stream);
hipError_t launch_gemm_mfma_i8(const GemmArgs& g, hipStream_t stream);
hipError_t launch_gemm_popcount(const GemmArgs& g, hipStream_t stream);
// Two-plane residual weights with K <= 64 (one word per plane row; g.N = 2 x outputs).
hipError_t launch_gemm_residual_word(const GemmArgs& g, hipStream_t stream);
hipError_t launch_gemv_popcount(const GemmArgs& g, hipStream_t stream);
// Two-plane residual weights, M <= 16 (g.N outputs, 2 g.N interleaved plane rows).
hipError_t launch_gemv_popcount_residual(const GemmArgs& g, hipStream_t stream);
hipError_t launch_gemv_mfma(const GemmArgs& g, hipStream_t stream);
// Workspace bytes launch_gemv_mfma uses for this shape when one is given (0: the
// shape runs without a cross-block split).
size_t gemv_mfma_workspace_bytes(int64_t M, int64_t N, int64_t K);
// Decode with the ternarization fused into the kernel: X holds M fp32 or bf16
// rows (row stride ldx elements); g's activation planes and scales are not
// read; o_* are optional outputs of the ternarization (NULL: not written).
hipError_t launch_gemv_fused(const GemmArgs& g, const void* X, Elt x_dt, int64_t ldx,
                             uint8_t* o_mask, uint8_t* o_sign, float* o_alpha, int32_t* o_nnz,
                             hipStream_t stream);
// The same with each row ternarized once, by one block, into exchange buffers
// (o_* when given, else workspace memory) that every block then stages; one
// launch.  ws: at least gemv_fused_xp_workspace_bytes, 256-byte aligned, its
// flag region zero before the first call (each call leaves it zero).  spin:
// polls of the row flags before a block ternarizes the rows itself.
// hipErrorNotSupported, with nothing launched, when the workspace is missing or
// short or the rows' staging does not fit one launch.
size_t gemv_fused_xp_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv_fused_xp(const GemmArgs& g, const void* X, Elt x_dt, int64_t ldx,
                                uint8_t* o_mask, uint8_t* o_sign, float* o_alpha,
                                int32_t* o_nnz, void* ws, size_t ws_bytes, int spin,
                                hipStream_t stream);
// The same for one activation row on the popcount decode kernel (gemm_popcount.hip);
// hipErrorNotSupported, with nothing launched, outside its fast path (M != 1,
// K % 8 != 0, K > 32768 (bf16) or 16384 (fp32), an odd number of 8-byte words
// per plane row, X not 16-byte aligned).
hipError_t launch_gemv_fused_row(const GemmArgs& g, const void* X, Elt x_dt, uint8_t* o_mask,
                                 uint8_t* o_sign, float* o_alpha, int32_t* o_nnz,
                                 hipStream_t stream);
// The library's own per-GPU scratch array (bwta_gemv_noalloc): its size, and the
// device address of the current device's copy (looked up, and its counter region
// cleared on `stream`, on the first call per device).
size_t scratch_bytes();
hipError_t scratch_workspace(void** ptr, hipStream_t stream);
// Two-plane residual weights, 2 <= M <= 16 (g.N outputs, 2 g.N interleaved plane rows).
hipError_t launch_gemv_mfma_residual(const GemmArgs& g, hipStream_t stream);

// Fused attention (attention.hip): ternary Q, K planes [heads * L, 16 bytes],
// binary V^T planes [heads * D, L / 8 bytes], O [heads * L, D].
struct AttentionArgs {
  int64_t heads, L, D;
  const uint8_t* q_mask;
  const uint8_t* q_sign;
  const float* q_alpha;
  const uint8_t* k_mask;
  const uint8_t* k_sign;
  const float* k_alpha;
  const uint8_t* v_sign;
  const float* v_alpha;
  float scale;
  void* O;
  Elt o_dt;
  float* p_out;      // optional
  uint8_t* p_mask;   // optional
  float* p_alpha;    // optional
  int32_t* p_nnz;    // optional
};

hipError_t launch_attention(const AttentionArgs& a, hipStream_t stream);

}  // namespace bwta
