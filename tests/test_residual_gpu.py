"""GPU parity of the two-plane residual binary weights (bwta_pack_weights_residual,
bwta_gemm_residual) against the oracle: planes, scales and products bit for bit.

BiLLM page ("BiLLM: Pushing the Limit of Post-Training Quantization for LLMs"),
Approach: salient weights are binarized with a residual, second-order
approximation; here every row gets the second plane, w ~ alpha1 s1 + alpha2 s2.
"""
import numpy as np
import pytest

from binary_ternary_matmul_amd import inputs
from tests.helpers import to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bw():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import binary_ternary_matmul_amd as b
    b.lib()
    return b


def interleave(p1, p2):
    """Plane row 64 (n // 32) + n % 32 holds plane 1 of row n, that + 32 plane 2."""
    n = np.arange(p1.shape[0])
    idx = 64 * (n // 32) + n % 32
    out = np.empty((2 * p1.shape[0],) + p1.shape[1:], p1.dtype)
    out[idx] = p1
    out[idx + 32] = p2
    return out


def expected_planes(oracle, W):
    s1, a1, s2, a2 = oracle.binarize_residual(W)
    return (s1, a1, s2, a2,
            interleave(oracle.pack_plane(s1, "sign"), oracle.pack_plane(s2, "sign")),
            interleave(a1, a2))


def _w(seed, N, K, bf16):
    rng = np.random.Generator(np.random.PCG64(seed))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    return inputs.f32_to_bf16_bits(w) if bf16 else w


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("N,K", [(32, 1), (32, 7), (64, 64), (96, 100), (32, 768),
                                 (256, 4096), (64, 11008), (32, 65536)])
def test_pack_residual(bw, oracle, N, K, bf16):
    W = _w(N * 7 + K, N, K, bf16)
    got = bw.bwta_pack_weights_residual(to_dev(W))
    *_, sign, alpha = expected_planes(oracle, W)
    assert (to_host(got.sign) == sign).all()
    assert (to_host(got.alpha).view(np.uint32) == alpha.view(np.uint32)).all()


def test_pack_residual_constant_rows(bw, oracle):
    """|w| constant along a row: plane 2 is all +1 and alpha2 = 0."""
    rng = np.random.default_rng(5)
    W = (np.where(rng.random((64, 300)) < 0.5, -1.0, 1.0) * 0.375).astype(np.float32)
    got = bw.bwta_pack_weights_residual(to_dev(W))
    *_, sign, alpha = expected_planes(oracle, W)
    assert (to_host(got.sign) == sign).all()
    assert (to_host(got.alpha) == alpha).all()


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(5, 64, 100), (3, 32, 65), (130, 96, 768), (128, 128, 256),
                                   (200, 320, 1000), (129, 4096, 4096),
                                   # K <= 64: one word per plane row (popcount kernel)
                                   (4, 32, 64), (1, 32, 1), (5, 64, 7), (130, 96, 33),
                                   (37, 320, 64), (300, 8192, 50)])
def test_gemm_residual(bw, oracle, M, N, K, out_dtype):
    x, w = inputs.random_linear(M * 3 + N + K, M, K, N)
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights_residual(to_dev(w))
    y = to_host(bw.bwta_gemm_residual(a, wp, out_dtype))
    t, aa, _ = oracle.ternarize(x)
    s1, a1, s2, a2 = oracle.binarize_residual(w)
    ref = oracle.scale_residual(oracle.matmul_i32(t, s1), oracle.matmul_i32(t, s2), aa, a1, a2)
    if out_dtype == "bf16":
        assert (y == oracle.to_bf16(ref)).all()
    else:
        assert (y.view(np.uint32) == ref.view(np.uint32)).all()


@pytest.mark.parametrize("K", [192, 40])
def test_gemm_residual_ldy(bw, oracle, K):
    """Output rows with a leading dimension larger than N; the gap is untouched."""
    import torch
    M, N = 70, 64
    x, w = inputs.random_linear(77, M, K, N)
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights_residual(to_dev(w))
    out = torch.full((M, N + 40), 7.0, device="cuda")
    bw.bwta_gemm_residual(a, wp, "f32", out=out[:, :N])
    got = to_host(out)
    t, aa, _ = oracle.ternarize(x)
    s1, a1, s2, a2 = oracle.binarize_residual(w)
    ref = oracle.scale_residual(oracle.matmul_i32(t, s1), oracle.matmul_i32(t, s2), aa, a1, a2)
    assert (got[:, :N].view(np.uint32) == ref.view(np.uint32)).all()
    assert (got[:, N:] == 7.0).all()


@pytest.mark.parametrize("M,N,K", [(2048, 4160, 1000), (2048, 6144, 1000)])
def test_gemm_residual_grid_rounds(bw, oracle, M, N, K):
    """16 x 65 plane tiles (4160 outputs, 8320 plane rows): 1024 tiles one per wave,
    the last 16 split over K in a second launch; 16 x 96 plane tiles (6144 outputs):
    512 blocks of paired waves and 512 blocks that split K in one launch.
    NaN-filled output, all rows on two columns of every 64-output tile."""
    import torch
    x, w = inputs.random_linear(4242, M, K, N)
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights_residual(to_dev(w))
    out = torch.full((M, N), float("nan"), device="cuda")
    y = to_host(bw.bwta_gemm_residual(a, wp, "f32", out=out))
    assert not np.isnan(y).any(), "outputs left unwritten"
    rng = np.random.default_rng(17)
    C = np.unique(np.concatenate([64 * j + rng.choice(64, size=2, replace=False)
                                  for j in range(N // 64)] + [[N - 1]]))
    t, aa, _ = oracle.ternarize(x)
    s1, a1, s2, a2 = oracle.binarize_residual(w)
    ref = oracle.scale_residual(oracle.matmul_i32(t, s1[C], threads=8),
                                oracle.matmul_i32(t, s2[C], threads=8), aa, a1[C], a2[C])
    assert (y[:, C].view(np.uint32) == ref.view(np.uint32)).all()


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(1, 32, 128), (1, 64, 100), (3, 96, 100), (4, 128, 8192),
                                   (7, 64, 2000), (16, 160, 4100), (16, 32, 28672),
                                   (2, 64, 129), (1, 32, 64), (5, 64, 1), (16, 4096, 65536),
                                   (13, 1024, 40000)])
def test_gemv_residual(bw, oracle, M, N, K, out_dtype):
    """Decode with two-plane weights: every output bit-exact.  M = 1 with 16-byte
    plane rows takes the popcount kernel, the rest the FP4 decode kernel (split K
    for long rows, raw activation staging for M = 16 at K = 65536)."""
    x, w = inputs.random_linear(M * 5 + N + K, M, K, N)
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights_residual(to_dev(w))
    y = to_host(bw.bwta_gemv_residual(a, wp, out_dtype))
    t, aa, _ = oracle.ternarize(x)
    s1, a1, s2, a2 = oracle.binarize_residual(w)
    ref = oracle.scale_residual(oracle.matmul_i32(t, s1), oracle.matmul_i32(t, s2), aa, a1, a2)
    if out_dtype == "bf16":
        assert (y == oracle.to_bf16(ref)).all()
    else:
        assert (y.view(np.uint32) == ref.view(np.uint32)).all()

