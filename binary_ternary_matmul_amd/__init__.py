"""Binary-weight x ternary-activation (BWTA) matrix products for AMD MI355X.

The compute lives in libbwta.so (hand-written HIP kernels for gfx950, C ABI in
include/bwta.h); this package is its Python binding.  Method: "BWTA: Accurate
and Efficient Binarized Transformer by Algorithm-Hardware Co-design", Abstract
(binary weights, ternary activations with tiny values projected to zero,
bit-packed binary/ternary MatMul for linear and attention operators).
"""
from ._binding import (AttentionProbs, BinaryPlanes, BwtaError, ResidualPlanes, TernaryPlanes,
                       bwta_attention, bwta_batched_gemm, bwta_gemm, bwta_gemm_residual,
                       bwta_gemm_workspace_size, bwta_gemv, bwta_gemv_residual,
                       bwta_gemv_workspace_size, bwta_pack_weights, bwta_pack_weights_residual,
                       bwta_gemv_fused, bwta_gemv_fused_workspace_size, bwta_gemv_noalloc,
                       bwta_ternarize_pack, lib, padded_k, row_bytes, set_fused_spin_limit,
                       workspace)

__all__ = ["AttentionProbs", "BinaryPlanes", "BwtaError", "ResidualPlanes", "TernaryPlanes",
           "bwta_attention", "bwta_batched_gemm", "bwta_gemm", "bwta_gemm_residual",
           "bwta_gemm_workspace_size", "bwta_gemv", "bwta_gemv_residual",
           "bwta_gemv_workspace_size", "bwta_pack_weights", "bwta_pack_weights_residual",
           "bwta_gemv_fused", "bwta_gemv_fused_workspace_size", "bwta_gemv_noalloc",
           "bwta_ternarize_pack", "lib", "padded_k", "row_bytes", "set_fused_spin_limit",
           "workspace"]
