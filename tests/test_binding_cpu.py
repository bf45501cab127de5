"""The Python binding's argument checks, on the CPU: every mismatch between the
tensors and the call (output dtype against out_dtype, plane dtype, shape or
stride, scale lengths, devices) raises ValueError before anything reaches the
library, so no kernel could write past an allocation.  Host tensors stand in
for device ones: the checks run before the device check, which is last."""
import os

import pytest
import torch


@pytest.fixture(scope="module")
def bw():
    from binary_ternary_matmul_amd import _binding, build
    if not os.path.exists(_binding.LIB_PATH):
        build.build()
    _binding.lib()
    return _binding


def tern(bw, rows, K, **over):
    rb = bw.row_bytes(K)
    parts = dict(mask=torch.zeros((rows, rb), dtype=torch.uint8),
                 sign=torch.zeros((rows, rb), dtype=torch.uint8),
                 alpha=torch.zeros(rows, dtype=torch.float32),
                 nnz=torch.zeros(rows, dtype=torch.int32))
    parts.update(over)
    return bw.TernaryPlanes(parts["mask"], parts["sign"], parts["alpha"], parts["nnz"], K)


def binr(bw, rows, K, **over):
    parts = dict(sign=torch.zeros((rows, bw.row_bytes(K)), dtype=torch.uint8),
                 alpha=torch.zeros(rows, dtype=torch.float32))
    parts.update(over)
    return bw.BinaryPlanes(parts["sign"], parts["alpha"], K)


def raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


@pytest.mark.parametrize("fn", ["bwta_gemm", "bwta_gemv"])
def test_product_out_checks(bw, fn):
    f = getattr(bw, fn)
    a, w = tern(bw, 4, 100), binr(bw, 8, 100)
    # a bf16 output with the default fp32 out_dtype: the kernel would write
    # 4-byte elements over a 2-byte allocation
    raises(lambda: f(a, w, out=torch.empty((4, 8), dtype=torch.bfloat16)), "dtype")
    raises(lambda: f(a, w, "i32", out=torch.empty((4, 8), dtype=torch.float32)), "dtype")
    raises(lambda: f(a, w, "bf16", out=torch.empty((4, 7), dtype=torch.bfloat16)), "x >= 8")
    raises(lambda: f(a, w, "f32", out=torch.empty((3, 8), dtype=torch.float32)), "x >= 8")
    raises(lambda: f(a, w, "f32", out=torch.empty((8, 4), dtype=torch.float32).t()), "stride")
    raises(lambda: f(a, w, "f32", out=torch.empty((4, 8), dtype=torch.float32, device="meta")),
           "meta")
    raises(lambda: f(a, w, "f64"), "out_dtype")
    raises(lambda: f(a, w, "f32", "fast"), "algo")
    # all arguments consistent: the last check is that they live on a GPU
    raises(lambda: f(a, w, "f32"), "device tensor")


def test_product_plane_checks(bw):
    K, rb = 100, bw.row_bytes(100)
    w = binr(bw, 8, K)
    raises(lambda: bw.bwta_gemm(tern(bw, 4, K, mask=torch.zeros((4, rb), dtype=torch.int8)), w),
           "uint8")
    raises(lambda: bw.bwta_gemm(tern(bw, 4, K, sign=torch.zeros((4, rb - 8), dtype=torch.uint8)),
                                w), "a.sign")
    wide = torch.zeros((4, 2 * rb), dtype=torch.uint8)[:, :rb]    # rows not back to back
    raises(lambda: bw.bwta_gemm(tern(bw, 4, K, mask=wide), w), "strides")
    raises(lambda: bw.bwta_gemm(tern(bw, 4, K, alpha=torch.zeros(3)), w), "a.alpha")
    raises(lambda: bw.bwta_gemm(tern(bw, 4, K, nnz=torch.zeros(4, dtype=torch.int64)), w), "a.nnz")
    raises(lambda: bw.bwta_gemm(tern(bw, 4, K), binr(bw, 8, K, alpha=torch.zeros(9))), "w.alpha")
    raises(lambda: bw.bwta_gemm(tern(bw, 4, K), binr(bw, 8, 200)), "K mismatch")


def test_batched_checks(bw):
    a, b = tern(bw, 8, 64), binr(bw, 16, 64)
    raises(lambda: bw.bwta_batched_gemm(2, a, 4, b, 8, 4, 8, "f32",
                                        out=torch.empty((2, 4, 8), dtype=torch.bfloat16)), "dtype")
    raises(lambda: bw.bwta_batched_gemm(3, a, 4, b, 8, 4, 8, "f32"), "past the rows")
    raises(lambda: bw.bwta_batched_gemm(2, a, 4, b, 8, 4, 8, "f32"), "device tensor")


def test_residual_and_attention_checks(bw):
    a, w = tern(bw, 4, 128), binr(bw, 64, 128)
    raises(lambda: bw.bwta_gemm_residual(a, bw.ResidualPlanes(w.sign, w.alpha, 128), "i32"),
           "out_dtype")
    raises(lambda: bw.bwta_gemm_residual(a, bw.ResidualPlanes(w.sign, w.alpha, 128), "f32",
                                         out=torch.empty((4, 32), dtype=torch.bfloat16)), "dtype")
    q = tern(bw, 512, 128)
    v = binr(bw, 128, 512)
    raises(lambda: bw.bwta_attention(q, q, v, 1, out=torch.empty((1, 512, 128),
                                                                 dtype=torch.bfloat16)), "dtype")
    raises(lambda: bw.bwta_attention(q, q, v, 1), "device tensor")
