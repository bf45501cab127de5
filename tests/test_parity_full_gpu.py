"""GPU parity at the benchmark workloads' full sizes, in the launch configuration
bench.py times (same entry points, algo and output dtype).

Every packed plane, alpha and nnz is compared in full, bit-exact, and so is
every product output:
  * the single linear (128 x 768 x 768), the BERT-base encoder linears
    (M = 4096), the LLaMA-7B prefill linears (M = 2048: each of the seven, and
    the stacked q/k/v and gate/up products the bench times), the decode GEMVs
    (M in {1, 4, 16} against 28672 x 8192 and 8192 x 28672 weights, and gate
    and up stacked into one 57344 x 8192 weight), both attention products and
    the two-plane residual products on the LLaMA-7B q and down linears: every
    int32 accumulator and every fp32/bf16 output against the oracle (its dense
    int8 loop over host threads), plus two properties any product of t in
    {-1, 0, +1} with s in {-1, +1} has: |acc| <= nnz and acc = nnz (mod 2);
  * the fused attention call (32 x 2048 x 128): O, the P planes, alpha_p and
    nnz_p of every head exactly on the kernel's own P, and P against the fp64
    softmax on all 32 heads (tests/test_attention_gpu.py states the checks).
"""
import os

import numpy as np
import pytest

from binary_ternary_matmul_amd import inputs
from tests.helpers import to_dev, to_host

pytestmark = pytest.mark.gpu

# the oracle's host threads (a GPU machine gives one GPU 16 cores)
THREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module")
def bw():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import binary_ternary_matmul_amd as b
    b.lib()
    return b


def _check_planes(bw, oracle, a, x):
    t, alpha, nnz = oracle.ternarize(x)
    assert (to_host(a.mask) == oracle.pack_plane(t, "mask")).all()
    assert (to_host(a.sign) == oracle.pack_plane(t, "sign")).all()
    assert (to_host(a.alpha).view(np.uint32) == alpha.view(np.uint32)).all()
    assert (to_host(a.nnz) == nnz).all()
    return t, alpha, nnz


def _check_weights(bw, oracle, wp, w, transpose=False):
    s, alpha = oracle.binarize(w, transpose=transpose)
    assert (to_host(wp.sign) == oracle.pack_plane(s, "sign")).all()
    assert (to_host(wp.alpha).view(np.uint32) == alpha.view(np.uint32)).all()
    return s, alpha


def _check_properties(acc, nnz):
    nz = nnz.astype(np.int64)[:, None]
    assert (np.abs(acc.astype(np.int64)) <= nz).all(), "|acc| > nnz"
    assert ((acc.astype(np.int64) - nz) % 2 == 0).all(), "acc and nnz differ in parity"


def _full_linear(bw, oracle, lin, x, algo, out_dtype):
    """One bench-shaped linear: planes, every accumulator and every output."""
    w = lin.w()
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights(to_dev(w))
    t, a_alpha, nnz = _check_planes(bw, oracle, a, x)
    s, w_alpha = _check_weights(bw, oracle, wp, w)
    del w
    acc = to_host(bw.bwta_gemm(a, wp, out_dtype="i32", algo=algo))
    _check_properties(acc, nnz)
    ref_acc = oracle.matmul_i32(t, s, threads=THREADS)
    del s
    bad = acc != ref_acc
    assert not bad.any(), f"{lin.name}: {int(bad.sum())} accumulators differ"
    del acc, bad
    y = to_host(bw.bwta_gemm(a, wp, out_dtype=out_dtype, algo=algo))
    ref_y = oracle.scale(ref_acc, a_alpha, w_alpha)
    if out_dtype == "bf16":
        bad = y != oracle.to_bf16(ref_y)
    else:
        bad = y.view(np.uint32) != ref_y.view(np.uint32)
    assert not bad.any(), f"{lin.name}: {int(bad.sum())} {out_dtype} outputs differ"


def test_full_single_linear(bw, oracle):
    """128 x 768 x 768, fp32 in and out: every output."""
    (lin,) = inputs.single_linear()
    x, w = lin.x(), lin.w()
    ref = oracle.linear(x, w, out="f32")
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights(to_dev(w))
    _check_planes(bw, oracle, a, x)
    _check_weights(bw, oracle, wp, w)
    acc = to_host(bw.bwta_gemm(a, wp, out_dtype="i32", algo="auto"))
    y = to_host(bw.bwta_gemm(a, wp, out_dtype="f32", algo="auto"))
    assert (acc == ref["acc"]).all()
    assert (y.view(np.uint32) == ref["y"].view(np.uint32)).all()


@pytest.mark.parametrize("i", range(len(inputs.BERT_SHAPES)))
def test_full_bert_encoder(bw, oracle, i):
    """BERT-base linears, M = 4096, fp32 in, bf16 out, algo auto (bench's call)."""
    lin = inputs.bert_encoder()[i]
    _full_linear(bw, oracle, lin, lin.x(), "auto", "bf16")


@pytest.mark.parametrize("i", range(len(inputs.LLAMA7B_SHAPES)))
def test_full_llama7b_prefill(bw, oracle, i):
    """LLaMA-7B prefill linears, M = 2048, bf16 in and out, algo mfma (bench's call)."""
    acts, lins = inputs.llama7b_prefill()
    lin = lins[i]
    x = acts[inputs.LLAMA7B_INPUTS[lin.name]]()
    _full_linear(bw, oracle, lin, x, "mfma", "bf16")


@pytest.mark.parametrize("name", ["qkv", "gate_up"])
def test_full_llama7b_stacked(bw, oracle, name):
    """The stacked products bench.py times (q/k/v weights as one [12288, 4096],
    gate/up as one [22016, 4096]), bf16 out, algo mfma: planes, accumulators and
    outputs in full (qkv runs as two launches, gate_up as one of three rounds)."""
    acts, prods = inputs.llama7b_products()
    lin = [p for p in prods if p.name == name][0]
    x = acts[inputs.LLAMA7B_INPUTS[name]]()
    _full_linear(bw, oracle, lin, x, "mfma", "bf16")


@pytest.mark.parametrize("shape", [n for n, _, _ in inputs.LLAMA70B_DECODE_SHAPES])
def test_full_llama70b_decode(bw, oracle, shape):
    """Decode GEMV at M = 1, 4, 16 on the full 70B-shaped weights, algo auto,
    fp32 out: every output."""
    lins = {M: [l for l in inputs.llama70b_decode(M) if l.name == shape][0] for M in (1, 4, 16)}
    w = lins[16].w()
    wp = bw.bwta_pack_weights(to_dev(w))
    s, w_alpha = _check_weights(bw, oracle, wp, w)
    del w
    for M, lin in lins.items():
        x = lin.x()
        a = bw.bwta_ternarize_pack(to_dev(x))
        t, a_alpha, nnz = _check_planes(bw, oracle, a, x)
        ref_acc = oracle.matmul_i32(t, s, threads=THREADS)
        acc = to_host(bw.bwta_gemv(a, wp, out_dtype="i32", algo="auto"))
        assert (acc == ref_acc).all(), f"M={M}: accumulators differ"
        y = to_host(bw.bwta_gemv(a, wp, out_dtype="f32", algo="auto"))
        ref_y = oracle.scale(ref_acc, a_alpha, w_alpha)
        assert (y.view(np.uint32) == ref_y.view(np.uint32)).all(), f"M={M}: outputs differ"



@pytest.mark.parametrize("shape", [n for n, _, _ in inputs.LLAMA70B_DECODE_SHAPES])
def test_full_llama70b_decode_fused(bw, oracle, shape):
    """The decode linear in one launch (bwta_gemv_fused: ternarize inside the
    decode kernel) on the full 70B-shaped weights, M = 1, 4, 16, bf16 in, fp32
    out, with the shared workspace: the kernel's planes, alpha and nnz, every
    accumulator and every output."""
    lins = {M: [l for l in inputs.llama70b_decode(M) if l.name == shape][0] for M in (1, 4, 16)}
    w = lins[16].w()
    wp = bw.bwta_pack_weights(to_dev(w))
    s, w_alpha = _check_weights(bw, oracle, wp, w)
    del w
    for M, lin in lins.items():
        x = lin.x()
        t, a_alpha, nnz = oracle.ternarize(x)
        acc, tp = bw.bwta_gemv_fused(to_dev(x), wp, "i32", planes=True)
        assert (to_host(tp.mask) == oracle.pack_plane(t, "mask")).all(), f"M={M}: mask"
        assert (to_host(tp.sign) == oracle.pack_plane(t, "sign")).all(), f"M={M}: sign"
        assert (to_host(tp.alpha).view(np.uint32) == a_alpha.view(np.uint32)).all()
        assert (to_host(tp.nnz) == nnz).all()
        ref_acc = oracle.matmul_i32(t, s, threads=THREADS)
        assert (to_host(acc) == ref_acc).all(), f"M={M}: accumulators differ"
        y = to_host(bw.bwta_gemv_fused(to_dev(x), wp, "f32"))
        ref_y = oracle.scale(ref_acc, a_alpha, w_alpha)
        assert (y.view(np.uint32) == ref_y.view(np.uint32)).all(), f"M={M}: outputs differ"

def test_full_llama70b_gate_up_stacked(bw, oracle):
    """Gate and up of one 70B MLP stacked into one [57344, 8192] weight (one decode
    launch for both), M = 1, 4, 16, algo auto, fp32 out: every output."""
    import torch
    lins = {M: [l for l in inputs.llama70b_decode(M) if l.name == "gate_up"][0] for M in (1, 4, 16)}
    wg = lins[16].w()
    wu = inputs.llama70b_up_weight()()
    pg, pu = bw.bwta_pack_weights(to_dev(wg)), bw.bwta_pack_weights(to_dev(wu))
    wp = bw.BinaryPlanes(torch.cat([pg.sign, pu.sign]), torch.cat([pg.alpha, pu.alpha]), pg.K)
    sg, ag = _check_weights(bw, oracle, pg, wg)
    su, au = _check_weights(bw, oracle, pu, wu)
    del wg, wu
    s = np.concatenate([sg, su])
    w_alpha = np.concatenate([ag, au])
    for M, lin in lins.items():
        x = lin.x()
        a = bw.bwta_ternarize_pack(to_dev(x))
        t, a_alpha, _ = _check_planes(bw, oracle, a, x)
        ref_acc = oracle.matmul_i32(t, s, threads=THREADS)
        acc = to_host(bw.bwta_gemv(a, wp, out_dtype="i32", algo="auto"))
        assert (acc == ref_acc).all(), f"M={M}: accumulators differ"
        y = to_host(bw.bwta_gemv(a, wp, out_dtype="f32", algo="auto"))
        ref_y = oracle.scale(ref_acc, a_alpha, w_alpha)
        assert (y.view(np.uint32) == ref_y.view(np.uint32)).all(), f"M={M}: outputs differ"


def test_full_attention(bw, oracle):
    """32 heads x 2048 x 128: Q K^T int32 scores in full; P V with P the oracle's
    softmax of the scaled scores (ternarized on the GPU) and V^T packed per
    channel in one launch from [L, H*D], fp32 out, in full."""
    import torch
    att = inputs.attention()
    H, L, D = att.heads, att.L, att.d
    q, k = att.q.reshape(H * L, D), att.k.reshape(H * L, D)
    qa = bw.bwta_ternarize_pack(to_dev(q))
    ka = bw.bwta_ternarize_pack(to_dev(k))
    tq, aq, _ = _check_planes(bw, oracle, qa, q)
    tk, ak, _ = _check_planes(bw, oracle, ka, k)
    scores = torch.empty((H, L, L), dtype=torch.int32, device="cuda")
    bw.bwta_batched_gemm(H, qa, L, ka, L, L, L, "i32", "auto", scores)
    got = to_host(scores)
    del scores
    P = np.empty((H * L, L), np.float32)
    for h in range(H):
        rows = slice(h * L, (h + 1) * L)
        ref = oracle.matmul_i32(tq[rows], tk[rows], threads=THREADS)
        assert (got[h] == ref).all(), f"scores of head {h} differ"
        P[rows] = oracle.attention_probs(ref, aq[rows], ak[rows], D)
    del got
    vf = np.ascontiguousarray(att.v.transpose(1, 0, 2).reshape(L, H * D))
    pa = bw.bwta_ternarize_pack(to_dev(P))
    vb = bw.bwta_pack_weights(to_dev(vf), transpose=True)
    tp, ap, _ = _check_planes(bw, oracle, pa, P)
    sv, av = _check_weights(bw, oracle, vb, vf, transpose=True)
    O = torch.empty((H, L, D), dtype=torch.float32, device="cuda")
    bw.bwta_batched_gemm(H, pa, L, vb, D, L, D, "f32", "auto", O)
    out = to_host(O)
    for h in range(H):
        rows, chans = slice(h * L, (h + 1) * L), slice(h * D, (h + 1) * D)
        acc = oracle.matmul_i32(tp[rows], sv[chans], threads=THREADS)
        ref = oracle.scale(acc, ap[rows], av[chans])
        assert (out[h].view(np.uint32) == ref.view(np.uint32)).all(), f"P V of head {h} differs"


def test_full_fused_attention(bw, oracle):
    """bwta_attention at 32 heads x 2048 x 128, fp32 out (bench's call)."""
    from tests.test_attention_gpu import check_attention
    check_attention(bw, oracle, 32, 2048, threads=THREADS)


@pytest.mark.parametrize("name", ["q", "down"])
def test_full_llama7b_residual(bw, oracle, name):
    """Two-plane residual weights for a LLaMA-7B prefill linear (M = 2048, bf16 in
    and out, bench's call): planes, scales and every output."""
    from tests.test_residual_gpu import expected_planes
    acts, lins = inputs.llama7b_prefill()
    lin = [l for l in lins if l.name == name][0]
    x = acts[inputs.LLAMA7B_INPUTS[lin.name]]()
    w = lin.w()
    a = bw.bwta_ternarize_pack(to_dev(x))
    wp = bw.bwta_pack_weights_residual(to_dev(w))
    s1, a1, s2, a2, sign, alpha = expected_planes(oracle, w)
    del w
    assert (to_host(wp.sign) == sign).all()
    assert (to_host(wp.alpha).view(np.uint32) == alpha.view(np.uint32)).all()
    t, aa, _ = _check_planes(bw, oracle, a, x)
    y = to_host(bw.bwta_gemm_residual(a, wp, "bf16"))
    acc1 = oracle.matmul_i32(t, s1, threads=THREADS)
    acc2 = oracle.matmul_i32(t, s2, threads=THREADS)
    ref = oracle.scale_residual(acc1, acc2, aa, a1, a2)
    bad = y != oracle.to_bf16(ref)
    assert not bad.any(), f"{name}: {int(bad.sum())} bf16 outputs differ"
