"""GPU parity of bwta_gemv_fused (decode linear with the ternarization fused into
the decode kernel) against the oracle.

The kernel's own ternarization (returned planes, alpha, nnz) must equal the
oracle's ternarize() of the same rows bit for bit, and so must the int32
accumulators, fp32 outputs and bf16 outputs computed from it.  Shapes cover
the vector load path (K a multiple of 8, aligned rows) and the element path
(ragged K, or a row stride that breaks 16-byte alignment), trees over fewer
lanes than a block (small K), the block-internal K split and the cross-block
split (with a workspace), and rows with zeros, signed zeros and outliers."""
import numpy as np
import pytest

from tests.helpers import to_dev, to_host
from tests.test_parity_gpu import _w, _x

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1000, 1024), (2, 513, 8192), (4, 300, 28672), (16, 300, 28672), (3, 77, 200),
          (1, 40, 65536), (5, 100, 100), (7, 257, 1000), (4, 33, 64), (1, 17, 1),
          (16, 1000, 28736), (9, 600, 36928),
          # the longest rows at M >= 2: the producing blocks read each row twice
          # (more than 8 runs of 8 values per thread), with the cross-block split
          (16, 300, 65536), (3, 513, 65536),
          # one row: the single-row kernel's launch shapes (4-, 8- and 16-wave blocks,
          # one, two and four 1 KiB chunks per weight row, ragged N and K) and plane
          # rows of an odd number of 8-byte words (12344, 4104: the general kernel)
          (1, 300, 28672), (1, 8200, 12360), (1, 2000, 16384), (1, 16500, 4168),
          (1, 8193, 8192), (1, 8200, 12344), (1, 16500, 4104)]


@pytest.fixture(scope="module")
def bw():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import binary_ternary_matmul_amd as b
    b.lib()
    return b


def _check(bw, oracle, x, w, Xd, ws):
    wp = bw.bwta_pack_weights(to_dev(w))
    t, alpha, nnz = oracle.ternarize(x)
    s, w_alpha = oracle.binarize(w)
    acc_ref = oracle.matmul_i32(t, s, threads=8)
    acc, tp = bw.bwta_gemv_fused(Xd, wp, "i32", planes=True, workspace=ws)
    assert (to_host(tp.mask) == oracle.pack_plane(t, "mask")).all(), "mask plane differs"
    assert (to_host(tp.sign) == oracle.pack_plane(t, "sign")).all(), "sign plane differs"
    assert (to_host(tp.alpha).view(np.uint32) == alpha.view(np.uint32)).all(), "alpha differs"
    assert (to_host(tp.nnz) == nnz).all(), "nnz differs"
    assert (to_host(acc) == acc_ref).all(), "accumulators differ"
    y_ref = oracle.scale(acc_ref, alpha, w_alpha)
    y = to_host(bw.bwta_gemv_fused(Xd, wp, "f32", workspace=ws))
    assert (y.view(np.uint32) == y_ref.view(np.uint32)).all(), "fp32 outputs differ"
    yb = to_host(bw.bwta_gemv_fused(Xd, wp, "bf16", workspace=ws))
    assert (yb == oracle.to_bf16(y_ref)).all(), "bf16 outputs differ"


@pytest.mark.parametrize("ws", [None, "auto"])
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemv_fused(bw, oracle, M, N, K, bf16, ws):
    x = _x(M * 31 + N + K, M, K, bf16)
    w = _w(N + K, N, K)
    _check(bw, oracle, x, w, to_dev(x), ws)


@pytest.mark.parametrize("pad", [8, 3])
def test_gemv_fused_row_stride(bw, oracle, pad):
    """Rows taken from a wider tensor (ldx = K + pad): pad 8 keeps bf16 rows
    16-byte aligned, pad 3 does not (element loads)."""
    M, N, K = 6, 700, 4096
    xw = _x(77 + pad, M, K + pad, True)
    x = np.ascontiguousarray(xw[:, :K])
    w = _w(5, N, K)
    _check(bw, oracle, x, w, to_dev(xw)[:, :K], "auto")


def test_gemv_fused_zero_rows(bw, oracle):
    """All-zero rows (nnz 0, alpha 0, outputs 0) next to normal ones."""
    M, N, K = 4, 300, 28672
    x = _x(9, M, K, True)
    x[1] = 0
    x[3] = 0x8000  # -0.0 in every column
    _check(bw, oracle, x, _w(10, N, K), to_dev(x), "auto")


# With the workspace ("auto" above) each row is ternarized once by one block and
# the other blocks wait for its flag.  The wait is bounded: a block that has polled
# the flags `spin` times ternarizes every row itself.  Spin 0 forces that path on
# every block (the kernel still ends normally; the rows are written several times
# with the same values).
@pytest.mark.parametrize("M,N,K", [(2, 513, 8192), (16, 300, 28672), (5, 100, 100),
                                   (9, 600, 36928), (1, 8200, 12344), (3, 77, 200),
                                   (4, 64, 65536)])
def test_gemv_fused_every_block_ternarizes(bw, oracle, M, N, K):
    x = _x(M * 7 + N, M, K, True)
    w = _w(N * 3 + K, N, K)
    bw.set_fused_spin_limit(0)
    try:
        _check(bw, oracle, x, w, to_dev(x), "auto")
    finally:
        bw.set_fused_spin_limit(-1)


def test_gemv_fused_calls_in_a_row(bw, oracle):
    """Calls of different M and K on one shared workspace: every call must find
    the row flags and the arrival counter zero, and leave them so."""
    import torch
    shapes = [(16, 1000, 8192), (4, 1000, 8192), (16, 520, 28672), (2, 64, 520), (16, 1000, 8192),
              (7, 3000, 4096)]
    for i, (M, N, K) in enumerate(shapes):
        x = _x(1000 + i, M, K, i % 2 == 0)
        w = _w(2000 + i, N, K)
        wp = bw.bwta_pack_weights(to_dev(w))
        t, alpha, nnz = oracle.ternarize(x)
        s, w_alpha = oracle.binarize(w)
        y_ref = oracle.scale(oracle.matmul_i32(t, s, threads=8), alpha, w_alpha)
        y = to_host(bw.bwta_gemv_fused(to_dev(x), wp, "f32", workspace="auto"))
        assert (y.view(np.uint32) == y_ref.view(np.uint32)).all(), f"call {i} {M}x{N}x{K} differs"
    # the split counters and the row flags (the first 8 KiB) are zero again
    ws = bw.workspace(torch.device("cuda", torch.cuda.current_device()), 0)
    assert int(ws[:8192].count_nonzero()) == 0, "counters or flags left non-zero"
