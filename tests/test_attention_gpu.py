"""GPU parity of the fused attention entry point (bwta_attention) against the oracle.

The kernel computes P with its own fp32 softmax, so P is compared with the
oracle's fp64 softmax within a bound derived from the fp32 arithmetic (below);
everything after P is exact and is compared bit for bit on the kernel's own P:
  * its P planes, alpha_p and nnz_p equal the oracle's ternarize() of that P;
  * O equals the oracle's product of those planes with V^T, scaled by the
    oracle's epilogue (fp32 bits, or bf16 bits for bf16 output);
  * the call without the optional outputs writes the same O.
Where the kernel's ternarization and the oracle's (of its own P) disagree, the
oracle's p must lie within the P bound of the row's threshold.

Bound on |P_gpu - P_ref| / P_ref (log2 units, x = (z - max z) log2 e, Z the
row's largest |z| log2 e, T = 16 values per lane): the scores u = S alpha_k and
the row factor a = alpha_q * scale * log2 e carry 1 and 3 roundings; each wave
exponentiates fma(a, u, -a m_w) against its own maximum m_w and the waves are
brought to the row maximum m by f_w = exp2(fma(a, m_w, -a m)), so the exponent
of e * f_w is off by at most (1.5 * 2^-23 + 2^-24) |x| (the factor a, and the two
fma roundings, whose arguments add up to |x|) plus 1.5 * 2^-23 Z (u and the two
products a * m rounded); exp2 turns that into a relative error ln 2 times as
large, and the two v_exp_f32 add about 1 ulp each; the sum (T sequential adds,
up to 7 tree levels, the products s_w f_w) and p = e * (f_w / s) add
(T + 12) * 2^-24.  The test allows twice the exponent term (the sum's terms
carry it too) plus those.
"""
import math

import numpy as np
import pytest

from binary_ternary_matmul_amd import inputs
from tests.helpers import to_dev, to_host

pytestmark = pytest.mark.gpu

D = 128
LOG2E = 1.0 / math.log(2.0)


@pytest.fixture(scope="module")
def bw():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import binary_ternary_matmul_amd as b
    b.lib()
    return b


def _operands(H, L, zero_q_rows=(), zero_k_rows=()):
    att = inputs.attention(H, L, D)
    q = att.q.reshape(H * L, D).copy()
    k = att.k.reshape(H * L, D).copy()
    q[list(zero_q_rows)] = 0
    k[list(zero_k_rows)] = 0
    vf = np.ascontiguousarray(att.v.transpose(1, 0, 2).reshape(L, H * D))
    return q, k, vf


def _p_bound(acc, aq, ak, head_dim, L):
    """Per-element relative bound on the kernel's P (see the module docstring)."""
    z = aq.astype(np.float64)[:, None] * ak.astype(np.float64)[None] * acc / math.sqrt(head_dim)
    x = (z - z.max(axis=1, keepdims=True)) * LOG2E
    Z = np.abs(z).max(axis=1, keepdims=True) * LOG2E
    T = 16
    return 2 * math.log(2) * (2.5 * 2.0 ** -23 * np.abs(x) + 1.5 * 2.0 ** -23 * Z
                              + 2 * 2.0 ** -23) + (T + 12) * 2.0 ** -24


def check_attention(bw, oracle, H, L, out_dtype="f32", head_dim=D, zero_q_rows=(),
                    zero_k_rows=(), threads=1, p_heads=None):
    """One call at heads x L x 128; O, the P planes, alpha_p and nnz_p of every
    head are checked, P against the fp64 softmax on the heads in p_heads (all by
    default).  Returns the number of P decisions that differ from the oracle's
    ternarization of its own P."""
    q, k, vf = _operands(H, L, zero_q_rows, zero_k_rows)
    scale = 1.0 / math.sqrt(head_dim)
    qa = bw.bwta_ternarize_pack(to_dev(q))
    ka = bw.bwta_ternarize_pack(to_dev(k))
    vb = bw.bwta_pack_weights(to_dev(vf), transpose=True)
    O, pr = bw.bwta_attention(qa, ka, vb, H, scale=scale, out_dtype=out_dtype, probs=True)
    O2 = bw.bwta_attention(qa, ka, vb, H, scale=scale, out_dtype=out_dtype)
    O, O2 = to_host(O), to_host(O2)
    P = to_host(pr.p)
    g_mask, g_alpha, g_nnz = to_host(pr.mask), to_host(pr.alpha), to_host(pr.nnz)

    tq, aq, _ = oracle.ternarize(q)
    tk, ak, _ = oracle.ternarize(k)
    sv, av = oracle.binarize(vf, transpose=True)
    # everything after P, exactly, on the kernel's P
    t, alpha, nnz = oracle.ternarize(P)
    assert (g_mask == oracle.pack_plane(t, "mask")).all(), "P planes differ from ternarize(P)"
    assert (g_alpha.view(np.uint32) == alpha.view(np.uint32)).all(), "alpha_p differs"
    assert (g_nnz == nnz).all(), "nnz_p differs"
    assert (O.view(np.uint16 if out_dtype == "bf16" else np.uint32) ==
            O2.view(np.uint16 if out_dtype == "bf16" else np.uint32)).all(), \
        "O differs without the optional outputs"
    flips = 0
    for h in range(H):
        rows, chans = slice(h * L, (h + 1) * L), slice(h * D, (h + 1) * D)
        acc = oracle.matmul_i32(t[rows], sv[chans], threads=threads)
        ref = oracle.scale(acc, alpha[rows], av[chans])
        if out_dtype == "bf16":
            assert (O[h] == oracle.to_bf16(ref)).all(), f"head {h}: O differs"
        else:
            assert (O[h].view(np.uint32) == ref.view(np.uint32)).all(), f"head {h}: O differs"
        if p_heads is not None and h not in p_heads:
            continue
        # P against the oracle's fp64 softmax of the exact scores
        S = oracle.matmul_i32(tq[rows], tk[rows], threads=threads)
        Pref = oracle.attention_probs(S, aq[rows], ak[rows], head_dim)
        bound = _p_bound(S, aq[rows], ak[rows], head_dim, L)
        err = np.abs(P[rows].astype(np.float64) - Pref)
        ok = err <= bound * Pref + 2.0 ** -126
        assert ok.all(), (f"head {h}: P off by up to {(err / np.maximum(Pref, 1e-300)).max():.3g} "
                          f"relative (bound {bound.max():.3g})")
        # decisions the oracle takes differently on its own P sit at the threshold
        tr, _, _ = oracle.ternarize(Pref)
        diff = tr != t[rows]
        if diff.any():
            thr = 0.5 * Pref.astype(np.float64).sum(axis=1, keepdims=True) / L
            near = np.abs(Pref - thr) <= 3 * bound * Pref + 2.0 ** -126
            assert near[diff].all(), f"head {h}: a P decision flips away from the threshold"
            flips += int(diff.sum())
    return flips


@pytest.mark.parametrize("H,L", [(2, 512), (1, 1024), (2, 2048)])
def test_attention_f32(bw, oracle, H, L):
    check_attention(bw, oracle, H, L)


def test_attention_bf16(bw, oracle):
    check_attention(bw, oracle, 1, 2048, out_dtype="bf16")


def test_attention_zero_rows(bw, oracle):
    """All-zero query rows (alpha_q = 0: uniform P, every key kept) and all-zero
    key rows (score 0 for every query)."""
    check_attention(bw, oracle, 1, 512, zero_q_rows=(0, 5, 17, 511), zero_k_rows=(3, 64, 500))


def test_attention_peaked(bw, oracle):
    """scale = 1 instead of 1 / sqrt(128): softmax rows close to one-hot."""
    check_attention(bw, oracle, 1, 1024, head_dim=1)


def test_attention_rejects_unsupported(bw):
    import torch
    q = bw.bwta_ternarize_pack(torch.zeros((256, 128), device="cuda"))
    v = bw.bwta_pack_weights(torch.zeros((256, 128), device="cuda"), transpose=True)
    with pytest.raises(bw.BwtaError):
        bw.bwta_attention(q, q, v, 1)   # L = 256 is not offered
