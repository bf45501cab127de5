"""Graph replays against eager calls.

bench.py times every figure as a HIP graph of calls replayed several times, so
the calls it times must give the same result on every replay as eagerly: the
cross-block K split's arrival counters, the fused decode's row flags and the
no-alloc entry point's scratch counters all have to come back to zero inside
each replay (nothing in the library records a memset).  One graph holds a
ternarize, the one-launch two-part prefill GEMM (16 x 96 tiles), a decode GEMV
that splits K across blocks through the shared workspace, the fused decode call
at M = 4 (each row ternarized once, flags in the workspace) and at M = 1 (the
one-row kernel), and bwta_gemv_noalloc.  Between replays the outputs are filled
with a sentinel and eager calls of other shapes use the same workspace and
scratch array; every replay must reproduce the eager outputs bit for bit.  The
eager outputs of the decode products are also checked against the oracle."""
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


def _x(seed, M, K):
    rng = np.random.Generator(np.random.PCG64(seed))
    return inputs.f32_to_bf16_bits(inputs.student_t(rng, (M, K), 3.0))


def _w(seed, N, K):
    rng = np.random.Generator(np.random.PCG64(seed))
    return inputs.normal(rng, (N, K), 0.02)


def test_graph_replays_match_eager(bw, oracle):
    import torch
    xp, wq = _x(1, 2048, 1000), _w(2, 12288, 1000)     # prefill: 1024 + 512 tiles, one launch
    xd, wd = _x(3, 16, 28672), _w(4, 520, 28672)       # decode M = 16: K split across blocks
    xf, wf = _x(5, 4, 8192), _w(6, 1000, 8192)         # fused decode, M = 4
    x1, w1 = _x(7, 1, 8192), _w(8, 3000, 8192)         # fused decode, one row
    d_xp, d_xd, d_xf, d_x1 = (to_dev(v) for v in (xp, xd, xf, x1))
    p_wq, p_wd, p_wf, p_w1 = (bw.bwta_pack_weights(to_dev(v)) for v in (wq, wd, wf, w1))
    dev = d_xp.device
    outs = {
        "prefill": torch.empty((2048, 12288), dtype=torch.bfloat16, device=dev),
        "gemv_split": torch.empty((16, 520), dtype=torch.int32, device=dev),
        "fused_m4": torch.empty((4, 1000), dtype=torch.float32, device=dev),
        "fused_m1": torch.empty((1, 3000), dtype=torch.float32, device=dev),
        "noalloc": torch.empty((16, 520), dtype=torch.int32, device=dev),
    }

    def step():
        a = bw.bwta_ternarize_pack(d_xp)
        bw.bwta_gemm(a, p_wq, "bf16", "mfma", out=outs["prefill"])
        ad = bw.bwta_ternarize_pack(d_xd)
        bw.bwta_gemv(ad, p_wd, "i32", "auto", out=outs["gemv_split"], workspace="auto")
        bw.bwta_gemv_fused(d_xf, p_wf, "f32", out=outs["fused_m4"])
        bw.bwta_gemv_fused(d_x1, p_w1, "f32", out=outs["fused_m1"])
        bw.bwta_gemv_noalloc(ad, p_wd, "i32", out=outs["noalloc"])

    assert bw.bwta_gemv_workspace_size(16, 520, 28672, "auto") > 0, "the shape must split K"
    # a shared workspace larger than every call below needs, so it never grows here
    # (a grown workspace leaves the old one allocated for the graphs that use it)
    bw.workspace(dev, 8 << 20)
    step()  # eager (also sizes the shared workspace and sets up the scratch array)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}

    # the eager decode outputs against the oracle
    td, _, _ = oracle.ternarize(xd)
    sd, _ = oracle.binarize(wd)
    acc = oracle.matmul_i32(td, sd, threads=8)
    assert (to_host(ref["gemv_split"]) == acc).all()
    assert (to_host(ref["noalloc"]) == acc).all()
    for x, w, key in ((xf, wf, "fused_m4"), (x1, w1, "fused_m1")):
        t, aa, _ = oracle.ternarize(x)
        s, ab = oracle.binarize(w)
        y = oracle.scale(oracle.matmul_i32(t, s, threads=8), aa, ab)
        assert (to_host(ref[key]).view(np.uint32) == y.view(np.uint32)).all(), key

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    # eager calls of other shapes on the same workspace and scratch array
    xo, wo = _x(9, 9, 4096), _w(10, 700, 4096)
    ao, p_wo = bw.bwta_ternarize_pack(to_dev(xo)), bw.bwta_pack_weights(to_dev(wo))
    for r in range(4):
        for k, v in outs.items():
            v.fill_(7 if v.dtype == torch.int32 else float("nan"))
        bw.bwta_gemv(ao, p_wo, "f32", "auto", workspace="auto")
        bw.bwta_gemv_fused(to_dev(xo), p_wo, "f32")
        bw.bwta_gemv_noalloc(ao, p_wo, "f32")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            same = torch.equal(v.view(torch.int16) if v.dtype == torch.bfloat16 else v.view(torch.int32),
                               ref[k].view(torch.int16) if v.dtype == torch.bfloat16
                               else ref[k].view(torch.int32))
            assert same, f"replay {r}: {k} differs from the eager result"
    # and the counter / flag region of the shared workspace is zero again
    ws = bw.workspace(dev, 8 << 20)
    assert int(ws[:8192].count_nonzero()) == 0
