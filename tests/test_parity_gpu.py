"""GPU parity: every libbwta kernel against the CPU oracle on the same seeded
inputs, at sizes that span several tiles and end in ragged tails.

Bar: packed planes, nnz and int32 accumulators bit-exact; alpha bit-exact (the
same pairwise tree); fp32 outputs within a relative error of 1e-5 (they are
expected to be bit-exact, since both sides evaluate fl32(acc * fl32(aa * ab)));
bf16 outputs equal after round-to-nearest-even.
"""
import numpy as np
import pytest

from binary_ternary_matmul_amd import inputs
from tests.helpers import to_dev, to_host

pytestmark = pytest.mark.gpu

REL_TOL = 1e-5


@pytest.fixture(scope="module")
def bw():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import binary_ternary_matmul_amd as b
    b.lib()
    return b


def _x(seed, M, K, bf16, nu=4.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = inputs.student_t(rng, (M, K), nu)
    x, _ = inputs.with_outlier_channels(x, rng, max(1, K // 100), 20.0)
    # a few exact zeros, signed zeros and a fully-zero row
    x[0, :: max(1, K // 7)] = 0.0
    if M > 2:
        x[2, :] = 0.0
    if M > 3:
        x[3, 1::3] = -0.0
    return inputs.f32_to_bf16_bits(x) if bf16 else x


def _w(seed, N, K, bf16=False):
    rng = np.random.Generator(np.random.PCG64(seed + 7))
    w = inputs.normal(rng, (N, K), 0.02)
    w[0, ::5] = 0.0
    if N > 1:
        w[1, ::3] = -0.0
    return inputs.f32_to_bf16_bits(w) if bf16 else w


def assert_close_f32(got, ref):
    ref = ref.astype(np.float64)
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > REL_TOL * np.abs(ref)
    assert not bad.any(), f"{bad.sum()} outputs beyond rel 1e-5; worst {err.max()}"


# ----------------------------------------------------------------------------
# ternarize_pack
# ----------------------------------------------------------------------------
# Row widths cover every launch plan of the row kernel: 16- and 32-lane rows,
# one wave of 1-8 groups, 8 groups on 2-4 waves (a partial last wave, K not a
# multiple of 8 on the element path, exactly 4 full waves), 4 groups on up to 16
# waves, and 8 re-reading groups on 16 waves.
TERN_SHAPES = [(1, 1), (3, 3), (5, 64), (7, 65), (9, 100), (33, 128), (17, 256), (16, 768),
               (12, 1000), (8, 2048), (6, 3072), (5, 4096), (4, 4097), (5, 6000), (3, 11008),
               (3, 12345), (2, 16384), (2, 16392), (2, 28672), (2, 65536)]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("M,K", TERN_SHAPES)
def test_ternarize_pack(bw, oracle, M, K, bf16):
    x = _x(100 + K, M, K, bf16)
    got = bw.bwta_ternarize_pack(to_dev(x))
    t, alpha, nnz = oracle.ternarize(x)
    assert (to_host(got.mask) == oracle.pack_plane(t, "mask")).all()
    assert (to_host(got.sign) == oracle.pack_plane(t, "sign")).all()
    assert (to_host(got.nnz) == nnz).all()
    assert (to_host(got.alpha).view(np.uint32) == alpha.view(np.uint32)).all()


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("K", [8, 4096, 11008, 65536])
def test_ternarize_pack_ties(bw, oracle, K, bf16):
    """Magnitudes equal to the threshold are dropped (|x| > thr keeps).  Each run
    of 8 is (2, 1.5, t, t, 0, 0, 0, 0) with t = 0.25 and signs varied, so every
    row sums exactly to K/2, mu = 0.5 and thr = 0.25 = t; rows scaled by powers
    of two keep the tie."""
    run = np.array([2.0, 1.5, 0.25, 0.25, 0.0, 0.0, 0.0, 0.0])
    rows = []
    for r in range(6):
        v = np.tile(run, K // 8) * 2.0 ** (r - 3)
        sgn = np.where((np.arange(K) * 7 + r) % 3 == 0, -1.0, 1.0)
        rows.append(v * sgn)
    x = np.array(rows, np.float32)
    if bf16:
        x = (x.view(np.uint32) >> 16).astype(np.uint16)
    got = bw.bwta_ternarize_pack(to_dev(x))
    t, alpha, nnz = oracle.ternarize(x)
    assert (nnz == 2 * (K // 8)).all(), "ties must be dropped"
    assert (to_host(got.mask) == oracle.pack_plane(t, "mask")).all()
    assert (to_host(got.sign) == oracle.pack_plane(t, "sign")).all()
    assert (to_host(got.nnz) == nnz).all()
    assert (to_host(got.alpha).view(np.uint32) == alpha.view(np.uint32)).all()


def test_ternarize_pack_row_stride(bw, oracle):
    import torch
    x = _x(5, 40, 300, False)
    big = np.zeros((40, 320), np.float32)
    big[:, :300] = x
    got = bw.bwta_ternarize_pack(to_dev(big)[:, :300])
    t, alpha, nnz = oracle.ternarize(x)
    assert (to_host(got.mask) == oracle.pack_plane(t, "mask")).all()
    assert (to_host(got.sign) == oracle.pack_plane(t, "sign")).all()
    assert (to_host(got.alpha) == alpha).all() and (to_host(got.nnz) == nnz).all()
    del torch


# ----------------------------------------------------------------------------
# pack_weights
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("N,K", [(1, 1), (3, 7), (70, 64), (33, 100), (130, 768), (9, 4096),
                                 (5, 11008), (4, 12345), (3, 28672)])
def test_pack_weights(bw, oracle, N, K, bf16):
    w = _w(N * 31 + K, N, K, bf16)
    got = bw.bwta_pack_weights(to_dev(w))
    s, alpha = oracle.binarize(w)
    assert (to_host(got.sign) == oracle.pack_plane(s, "sign")).all()
    assert (to_host(got.alpha).view(np.uint32) == alpha.view(np.uint32)).all()


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("L,C", [(2048, 128), (100, 70), (64, 1), (1000, 72), (520, 64),
                                 (300, 8), (4096, 24), (65536, 8)])
def test_pack_weights_columns(bw, oracle, L, C, bf16):
    """V^T packing: the columns of a row-major [L, C] matrix become rows.  The
    staged kernel takes C a multiple of the 16-byte vector and L >= 512 (bf16)
    or 256 (fp32) - including ragged L and a partial last block of columns;
    the others take the per-lane kernel."""
    v = _w(L + C, L, C, bf16)
    got = bw.bwta_pack_weights(to_dev(v), transpose=True)
    s, alpha = oracle.binarize(v, transpose=True)
    assert (to_host(got.sign) == oracle.pack_plane(s, "sign")).all()
    assert (to_host(got.alpha) == alpha).all()


# ----------------------------------------------------------------------------
# products
# ----------------------------------------------------------------------------
GEMM_SHAPES = [(1, 1, 1), (5, 3, 64), (17, 33, 65), (128, 128, 256), (130, 260, 200),
               (40, 50, 128), (33, 70, 192), (129, 257, 320), (70, 90, 448),
               (257, 129, 1000), (128, 768, 768), (300, 130, 4096), (64, 300, 11008),
               (200, 100, 28672 + 64),
               # K split over two waves with one or two 256-k steps each, the last
               # step holding the row end (520: a 16-byte window straddles it)
               (150, 140, 520), (64, 1000, 330)]


def _linear_case(oracle, M, N, K, bf16=False):
    x = _x(M * 1000 + N + K, M, K, bf16)
    w = _w(M + N * 7 + K, N, K)
    ref = oracle.linear(x, w, out="bf16")
    return x, w, ref


@pytest.mark.parametrize("algo", ["mfma", "mfma_i8", "popcount"])
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm(bw, oracle, M, N, K, algo):
    x, w, ref = _linear_case(oracle, M, N, K)
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights(to_dev(w))
    acc = to_host(bw.bwta_gemm(a, wp, out_dtype="i32", algo=algo))
    assert (acc == ref["acc"]).all(), f"{(acc != ref['acc']).sum()} accumulators differ"
    y = to_host(bw.bwta_gemm(a, wp, out_dtype="f32", algo=algo))
    assert_close_f32(y, ref["y"])
    assert (y.view(np.uint32) == ref["y"].view(np.uint32)).all()
    yb = to_host(bw.bwta_gemm(a, wp, out_dtype="bf16", algo=algo))
    assert (yb == ref["y_bf16"]).all()


def test_gemm_ldy(bw, oracle):
    import torch
    M, N, K = 70, 90, 300
    x, w, ref = _linear_case(oracle, M, N, K)
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights(to_dev(w))
    for algo in ["mfma", "mfma_i8", "popcount"]:
        out = torch.full((M, 100), -7.0, device="cuda")
        bw.bwta_gemm(a, wp, out_dtype="f32", algo=algo, out=out)
        o = to_host(out)
        assert (o[:, :N] == ref["y"]).all() and (o[:, N:] == -7.0).all()



@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_gemm_ldy_complete_tiles(bw, oracle, out_dtype):
    """Complete 128 x 128 tiles (M, N multiples of 128) into rows whose pitch is
    not a multiple of 16 bytes (ldy = 385): the tiles must not take the 16-byte
    staged stores; every output and the gap columns are checked."""
    import torch
    M, N, K, ldy = 256, 384, 300, 385
    x, w, ref = _linear_case(oracle, M, N, K)
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights(to_dev(w))
    tdt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    for algo in ["mfma", "mfma_i8", "popcount"]:
        out = torch.full((M, ldy), -7.0, dtype=tdt, device="cuda")
        bw.bwta_gemm(a, wp, out_dtype=out_dtype, algo=algo, out=out[:, :N])
        o = to_host(out)
        want = oracle.to_bf16(ref["y"]) if out_dtype == "bf16" else ref["y"]
        sentinel = to_host(torch.full((1,), -7.0, dtype=tdt))[0]
        assert (o[:, :N].view(want.dtype) == want).all(), algo
        assert (o[:, N:] == sentinel).all(), algo

# Grids of more 128 x 128 output tiles than the chip's 1024 SIMDs: whole rounds
# run one tile per wave over all of K, the last partial round (at most 512
# tiles) splits each tile's K range over two waves - in one launch of two-wave
# blocks (paired waves for the whole rounds) where the column count is even and
# the whole rounds end on whole column pairs, else as a second launch.  Outputs start as a sentinel, every output is checked against the
# properties |acc| <= nnz and acc = nnz (mod 2), and all rows against the oracle
# on two columns of every 128-column tile.
# Grids that stay one unsplit launch (a partial round above 512 tiles, or fewer
# than 4 steps of K) run their waves in pairs on adjacent column tiles sharing A;
# an odd column count leaves the last pair's second wave without a tile.
GRID_SHAPES = [(2048, 8300, 1000),   # 16 x 65 tiles = 1024 + 16; ragged N, ragged K
               (1900, 8960, 1536),   # 15 x 70 tiles = 1024 + 26; ragged M
               (1000, 24654, 300),   # 8 x 193 tiles = 1024 + 520: pairs, odd columns
               (1100, 16500, 500),   # 9 x 129 tiles, 2 steps of K: pairs, odd columns
               (2048, 12288, 1000),  # 16 x 96 = 1024 + 512 in one launch; ragged K
               (2000, 12288, 2000),  # the same grid, ragged M, 8 steps of K
               (1536, 16384, 800),   # 12 x 128 in one launch: bands of 8 and 4 rows
               (1024, 20480, 1100),  # 8 x 160 = 1024 + 256 in one launch
               (2048, 12200, 1000)]  # 16 x 96 in one launch, ragged last column


def _grid_columns(N, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    cols = [min(N - 1, 128 * j + int(c)) for j in range((N + 127) // 128)
            for c in rng.choice(128, size=2, replace=False)]
    return np.unique(np.array(cols + [N - 1], dtype=np.int64))


@pytest.mark.parametrize("M,N,K", GRID_SHAPES)
def test_gemm_grid_rounds(bw, oracle, M, N, K):
    import torch
    x = _x(M + N + K, M, K, True)
    w = _w(N + 3 * K, N, K)
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights(to_dev(w))
    t, aa, nnz = oracle.ternarize(x)
    s, ab = oracle.binarize(w)
    C = _grid_columns(N, M + K)
    ref_acc = oracle.matmul_i32(t, s[C], threads=8)
    acc = torch.full((M, N), 0x7FFFFFFF, dtype=torch.int32, device="cuda")
    acc = to_host(bw.bwta_gemm(a, wp, out_dtype="i32", algo="mfma", out=acc)).astype(np.int64)
    nz = nnz.astype(np.int64)[:, None]
    assert (np.abs(acc) <= nz).all() and ((acc - nz) % 2 == 0).all(), "an output breaks |acc| <= nnz"
    assert (acc[:, C] == ref_acc).all(), f"{(acc[:, C] != ref_acc).sum()} accumulators differ"
    y = torch.full((M, N), float("nan"), device="cuda")
    y = to_host(bw.bwta_gemm(a, wp, out_dtype="f32", algo="mfma", out=y))
    assert not np.isnan(y).any(), "outputs left unwritten"
    ref = oracle.scale(ref_acc, aa, ab[C])
    assert (y[:, C].view(np.uint32) == ref.view(np.uint32)).all()
    yb = to_host(bw.bwta_gemm(a, wp, out_dtype="bf16", algo="mfma"))
    assert (yb[:, C] == oracle.to_bf16(ref)).all()


@pytest.mark.parametrize("ws", [None, "auto"])
@pytest.mark.parametrize("algo", ["popcount", "mfma", "mfma_i8", "auto"])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 16])
@pytest.mark.parametrize("N,K", [(1000, 1024), (513, 8192), (300, 28672), (77, 200)])
def test_gemv(bw, oracle, M, N, K, algo, ws):
    """ws=None: no workspace (K split inside blocks); "auto": the shared
    workspace, which splits K across blocks where 513 x 8192 and 300 x 28672
    would split it inside a block."""
    x, w, ref = _linear_case(oracle, M, N, K, bf16=True)
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights(to_dev(w))
    acc = to_host(bw.bwta_gemv(a, wp, out_dtype="i32", algo=algo, workspace=ws))
    assert (acc == ref["acc"]).all()
    y = to_host(bw.bwta_gemv(a, wp, out_dtype="f32", algo=algo, workspace=ws))
    assert (y.view(np.uint32) == ref["y"].view(np.uint32)).all()


@pytest.mark.parametrize("ws", [None, "auto"])
@pytest.mark.parametrize("algo", ["mfma", "popcount"])
@pytest.mark.parametrize("M,N,K", [(16, 40, 65536), (13, 21, 40000), (9, 600, 36928),
                                   (16, 4100, 17000), (6, 33, 64), (2, 17, 129)])
def test_gemv_launch_paths(bw, oracle, M, N, K, algo, ws):
    """Decode shapes that take the other launch paths of the FP4 GEMV.  Without
    a workspace: raw activation planes (expanded operands do not fit in LDS),
    activation rows split over several launches (K = 65536 at M = 16), a K split
    over up to 8 waves for few weight rows, ragged K and N, and tiny K.  With
    one, the in-block K splits become cross-block splits of up to 8 ranges."""
    x, w, ref = _linear_case(oracle, M, N, K, bf16=True)
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights(to_dev(w))
    acc = to_host(bw.bwta_gemv(a, wp, out_dtype="i32", algo=algo, workspace=ws))
    assert (acc == ref["acc"]).all()
    y = to_host(bw.bwta_gemv(a, wp, out_dtype="bf16", algo=algo, workspace=ws))
    assert (y == ref["y_bf16"]).all()


def test_gemv_workspace_reuse(bw, oracle):
    """One caller-owned workspace through several calls: the first shape (ragged
    K = 28736, 57 chunks in 4 ranges) twice, then a smaller one, then bwta_gemm
    (AUTO sends M <= 16 to the same kernel).  Every output is checked, and the
    per-tile counters at the front of the workspace read zero after each call
    (a later call with more tiles must not find an earlier call's partials where
    its counters are)."""
    import torch
    cases = [(16, 1000, 28736), (16, 1000, 28736), (9, 300, 9000), (8, 513, 16384),
             (16, 4100, 17000)]   # more tiles than any call before it
    need = max(bw.bwta_gemv_workspace_size(M, N, K) for M, N, K in cases)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, (M, N, K) in enumerate(cases):
        assert bw.bwta_gemv_workspace_size(M, N, K) > 0, (M, N, K)
        x, w, ref = _linear_case(oracle, M, N, K, bf16=True)
        a = bw.bwta_ternarize_pack(to_dev(x))
        wp = bw.bwta_pack_weights(to_dev(w))
        fn = bw.bwta_gemm if i >= 3 else bw.bwta_gemv
        acc = to_host(fn(a, wp, out_dtype="i32", algo="auto", workspace=ws))
        assert (acc == ref["acc"]).all(), f"call {i}: accumulators differ"
        y = to_host(fn(a, wp, out_dtype="f32", algo="auto", workspace=ws))
        assert (y.view(np.uint32) == ref["y"].view(np.uint32)).all(), f"call {i}: outputs differ"
        tiles = (N + 15) // 16
        assert (to_host(ws[:4 * tiles].view(torch.int32)) == 0).all(), f"call {i}: counters left"


def test_gemv_ldy(bw, oracle):
    """Outputs with a leading dimension larger than N keep the gap untouched."""
    import torch
    M, N, K = 5, 90, 3000
    x, w, ref = _linear_case(oracle, M, N, K, bf16=True)
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights(to_dev(w))
    for algo in ["mfma", "popcount"]:
        out = torch.full((M, 97), -7.0, device="cuda")
        bw.bwta_gemv(a, wp, out_dtype="f32", algo=algo, out=out[:, :N])
        o = to_host(out)
        assert (o[:, :N].view(np.uint32) == ref["y"].view(np.uint32)).all()
        assert (o[:, N:] == -7.0).all()


@pytest.mark.parametrize("algo", ["mfma", "mfma_i8", "popcount"])
@pytest.mark.parametrize("H,L,D", [(3, 130, 128), (2, 257, 64), (4, 256, 100)])
def test_batched_ternary_ternary(bw, oracle, H, L, D, algo):
    rng = np.random.Generator(np.random.PCG64(H * L + D))
    q = inputs.f32_to_bf16_bits(rng.standard_normal((H * L, D), dtype=np.float32))
    k = inputs.f32_to_bf16_bits(rng.standard_normal((H * L, D), dtype=np.float32) * 1.5)
    qa = bw.bwta_ternarize_pack(to_dev(q))
    ka = bw.bwta_ternarize_pack(to_dev(k))
    got = to_host(bw.bwta_batched_gemm(H, qa, L, ka, L, L, L, out_dtype="i32", algo=algo))
    tq, _, _ = oracle.ternarize(q)
    tk, _, _ = oracle.ternarize(k)
    for h in range(H):
        ref = oracle.matmul_i32(tq[h * L:(h + 1) * L], tk[h * L:(h + 1) * L])
        assert (got[h] == ref).all(), f"head {h}"


def test_batched_grid_pairs(bw, oracle):
    """5 heads of L = 1913: 15 x 15 tiles per head, 1125 in all, so one unsplit
    launch with paired waves and an odd column count; sentinel-filled output,
    every score checked."""
    import torch
    H, L, D = 5, 1913, 128
    rng = np.random.Generator(np.random.PCG64(H * L + D))
    q = inputs.f32_to_bf16_bits(rng.standard_normal((H * L, D), dtype=np.float32))
    k = inputs.f32_to_bf16_bits(rng.standard_normal((H * L, D), dtype=np.float32) * 1.5)
    qa = bw.bwta_ternarize_pack(to_dev(q))
    ka = bw.bwta_ternarize_pack(to_dev(k))
    out = torch.full((H, L, L), 0x7FFFFFFF, dtype=torch.int32, device="cuda")
    got = to_host(bw.bwta_batched_gemm(H, qa, L, ka, L, L, L, out_dtype="i32", algo="mfma",
                                       out=out))
    tq, _, _ = oracle.ternarize(q)
    tk, _, _ = oracle.ternarize(k)
    for h in range(H):
        ref = oracle.matmul_i32(tq[h * L:(h + 1) * L], tk[h * L:(h + 1) * L], threads=8)
        assert (got[h] == ref).all(), f"head {h}"



@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_batched_grid_pairs_scaled(bw, oracle, out_dtype):
    """The paired-wave grid of test_batched_grid_pairs (5 x 1913 x 1913, ternary
    B, odd column count) with the scaled epilogue: each wave of a pair uses its
    own column scales; every output compared bit for bit."""
    import torch
    H, L, D = 5, 1913, 128
    rng = np.random.Generator(np.random.PCG64(H * L + D + 1))
    q = inputs.f32_to_bf16_bits(rng.standard_normal((H * L, D), dtype=np.float32))
    k = inputs.f32_to_bf16_bits(rng.standard_normal((H * L, D), dtype=np.float32) * 0.7)
    qa = bw.bwta_ternarize_pack(to_dev(q))
    ka = bw.bwta_ternarize_pack(to_dev(k))
    tdt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.full((H, L, L), float("nan"), dtype=tdt, device="cuda")
    got = to_host(bw.bwta_batched_gemm(H, qa, L, ka, L, L, L, out_dtype=out_dtype, algo="mfma",
                                       out=out))
    tq, aq, _ = oracle.ternarize(q)
    tk, ak, _ = oracle.ternarize(k)
    for h in range(H):
        rows = slice(h * L, (h + 1) * L)
        ref = oracle.scale(oracle.matmul_i32(tq[rows], tk[rows], threads=8), aq[rows], ak[rows])
        if out_dtype == "bf16":
            assert (got[h] == oracle.to_bf16(ref)).all(), f"head {h}"
        else:
            assert (got[h].view(np.uint32) == ref.view(np.uint32)).all(), f"head {h}"

@pytest.mark.parametrize("out_dtype", ["i32", "f32"])
def test_batched_two_part_ternary(bw, oracle, out_dtype):
    """One batch of a ternary x ternary product on a 16 x 96 tile grid (2048 x
    12288, K = 1000): the one-launch two-part grid with ternary B planes (paired
    waves on 1024 tiles, K split in two on the last 512); sentinel-filled output,
    all rows on two columns of every tile, every score within |acc| <= nnz."""
    import torch
    M, N, K = 2048, 12288, 1000
    rng = np.random.Generator(np.random.PCG64(M + N + K))
    q = inputs.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    k = inputs.f32_to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32) * 1.3)
    qa = bw.bwta_ternarize_pack(to_dev(q))
    ka = bw.bwta_ternarize_pack(to_dev(k))
    tdt = torch.int32 if out_dtype == "i32" else torch.float32
    fill = 0x7FFFFFFF if out_dtype == "i32" else float("nan")
    out = torch.full((1, M, N), fill, dtype=tdt, device="cuda")
    got = to_host(bw.bwta_batched_gemm(1, qa, M, ka, N, M, N, out_dtype=out_dtype, algo="mfma",
                                       out=out))[0]
    tq, aq, nq = oracle.ternarize(q)
    tk, ak, _ = oracle.ternarize(k)
    C = _grid_columns(N, 5)
    ref = oracle.matmul_i32(tq, tk[C], threads=8)
    if out_dtype == "i32":
        acc = got.astype(np.int64)
        nz = nq.astype(np.int64)[:, None]
        assert (np.abs(acc) <= nz).all(), "a score breaks |acc| <= nnz"  # (no parity rule: B is ternary)
        assert (acc[:, C] == ref).all(), f"{(acc[:, C] != ref).sum()} scores differ"
    else:
        assert not np.isnan(got).any(), "outputs left unwritten"
        want = oracle.scale(ref, aq, ak[C])
        assert (got[:, C].view(np.uint32) == want.view(np.uint32)).all()


def test_pack_weights_columns_all_heads(bw, oracle):
    """V laid out [L, H*D]: one call packs V^T of every head (row h*D + d)."""
    rng = np.random.Generator(np.random.PCG64(3))
    H, L, D = 5, 2048, 128
    v = inputs.f32_to_bf16_bits(rng.standard_normal((L, H * D), dtype=np.float32))
    got = bw.bwta_pack_weights(to_dev(v), transpose=True)
    s, alpha = oracle.binarize(v, transpose=True)
    assert (to_host(got.sign) == oracle.pack_plane(s, "sign")).all()
    assert (to_host(got.alpha) == alpha).all()


@pytest.mark.parametrize("algo", ["mfma", "mfma_i8", "popcount"])
@pytest.mark.parametrize("H,L,D", [(2, 300, 128), (3, 256, 64)])
def test_batched_ternary_binary(bw, oracle, H, L, D, algo):
    """P V: ternary P [L, L] per head times binary V^T [D, L] per head."""
    import torch
    rng = np.random.Generator(np.random.PCG64(H + L + D))
    P = rng.dirichlet(np.ones(L), size=H * L).astype(np.float32)         # rows sum to 1
    V = inputs.f32_to_bf16_bits(rng.standard_normal((H, L, D), dtype=np.float32))
    pa = bw.bwta_ternarize_pack(to_dev(P))
    vt_sign = torch.empty((H * D, bw.row_bytes(L)), dtype=torch.uint8, device="cuda")
    vt_alpha = torch.empty(H * D, dtype=torch.float32, device="cuda")
    Vd = to_dev(V)
    for h in range(H):
        vp = bw.bwta_pack_weights(Vd[h], transpose=True)
        vt_sign[h * D:(h + 1) * D] = vp.sign
        vt_alpha[h * D:(h + 1) * D] = vp.alpha
    vb = bw.BinaryPlanes(vt_sign, vt_alpha, L)
    got = to_host(bw.bwta_batched_gemm(H, pa, L, vb, D, L, D, out_dtype="f32", algo=algo))
    tp, ap, _ = oracle.ternarize(P)
    for h in range(H):
        s, av = oracle.binarize(V[h], transpose=True)
        acc = oracle.matmul_i32(tp[h * L:(h + 1) * L], s)
        ref = oracle.scale(acc, ap[h * L:(h + 1) * L], av)
        assert (got[h].view(np.uint32) == ref.view(np.uint32)).all(), f"head {h}"


def test_empty_and_degenerate(bw, oracle):
    import torch
    # zero rows: no-op
    X = torch.zeros((0, 64), device="cuda")
    got = bw.bwta_ternarize_pack(X)
    assert got.mask.shape == (0, 8)
    # all-zero activations: every output is 0
    x = np.zeros((5, 200), np.float32)
    w = _w(1, 9, 200)
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights(to_dev(w))
    assert (to_host(a.nnz) == 0).all() and (to_host(a.alpha) == 0).all()
    for algo in ["mfma", "mfma_i8", "popcount"]:
        assert (to_host(bw.bwta_gemm(a, wp, algo=algo)) == 0).all()
        assert (to_host(bw.bwta_gemv(a, wp, algo=algo)) == 0).all()
