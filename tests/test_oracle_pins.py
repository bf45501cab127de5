"""Pins for the CPU oracle: closed forms, hand-derived examples, library routines,
brute force and invariants.  CPU only.

The method is the binary-weight x ternary-activation product of "BWTA: Accurate
and Efficient Binarized Transformer by Algorithm-Hardware Co-design", Abstract
(binary weights; ternary activations with tiny values projected to zero; a
bit-packed binary/ternary MatMul).  The threshold 0.5*mean|x|, the scales and the
pairwise-tree order are the library's definition of what the page leaves open;
each test below pins one part of that definition against something other than
the oracle's own code.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
F = np.float32
TWO24 = float(2 ** 24)


def unpack_bits(plane: np.ndarray, K: int) -> np.ndarray:
    """Independent unpacking through numpy's own bit routine (LSB-first)."""
    return np.unpackbits(plane, axis=1, bitorder="little")[:, :K].astype(np.int8)


# ----------------------------------------------------------------------------
# tree sum
# ----------------------------------------------------------------------------

def test_tree_order_power_of_two(oracle):
    # (2^24 + 1) rounds to 2^24 (tie to even), (1 + 1) = 2, so the tree gives
    # 2^24 + 2; a left-to-right sum would give 2^24.
    assert oracle.tree_sum([TWO24, 1, 1, 1]) == F(TWO24 + 2)
    assert oracle.tree_sum([1, TWO24, 1, 1]) == F(TWO24 + 2)
    # 8 leaves: level 1 -> 2^24, 2, 2, 2; level 2 -> 2^24 + 2, 4; level 3 -> 2^24 + 6.
    assert oracle.tree_sum([TWO24] + [1] * 7) == F(TWO24 + 6)


def test_tree_zero_padded_shape(oracle):
    # K = 3 is padded to 4 leaves: (2^24 + 1) + (1 + 0) = 2^24 (two ties to even).
    # A split-at-floor(n/2) recursion would give 2^24 + (1 + 1) = 2^24 + 2.
    assert oracle.tree_sum([TWO24, 1, 1]) == F(TWO24)
    # K = 5 -> 8 leaves: ((2^24+1)+(1+1)) + ((1+0)+(0+0)) = (2^24+2) + 1, a tie
    # between 2^24+2 (odd significand) and 2^24+4 (even) -> 2^24+4.
    assert oracle.tree_sum([TWO24, 1, 1, 1, 1]) == F(TWO24 + 4)


def test_tree_exact_on_small_integers(oracle):
    # Every partial sum of small non-negative integers is exact in fp32.
    rng = np.random.default_rng(1)
    for n in [1, 2, 3, 5, 63, 64, 65, 100, 1000, 4097]:
        v = rng.integers(0, 100, size=n).astype(np.float32)
        assert oracle.tree_sum(v) == F(int(v.astype(np.int64).sum()))
    assert oracle.tree_sum(np.ones(28672, np.float32)) == F(28672)


def test_tree_padding_invariance(oracle):
    # A perfect tree over a longer zero-padded power of two has the same root.
    rng = np.random.default_rng(2)
    for n in [3, 7, 64, 100, 777]:
        v = np.abs(rng.standard_t(3, size=n)).astype(np.float32)
        base = oracle.tree_sum(v)
        for extra in [1, 5, 64, 1000]:
            assert oracle.tree_sum(np.concatenate([v, np.zeros(extra, np.float32)])) == base


def test_tree_matches_recursive_halving(oracle):
    # For a power-of-two length the tree is classic recursive halving.
    def rec(v):
        if len(v) == 1:
            return F(v[0])
        h = len(v) // 2
        return F(rec(v[:h]) + rec(v[h:]))

    rng = np.random.default_rng(3)
    for n in [1, 2, 4, 16, 128, 1024]:
        v = rng.standard_normal(n).astype(np.float32)
        assert oracle.tree_sum(v) == rec(list(v))


def test_tree_error_bound(oracle):
    # Pairwise summation: |tree - exact| <= ceil(log2 P) * u * sum|v| (u = 2^-24).
    rng = np.random.default_rng(4)
    for n in [3, 100, 768, 4096, 11008]:
        v = np.abs(rng.standard_t(3, size=n)).astype(np.float32)
        exact = sum(Fraction(float(x)) for x in v)
        P = 1 << (n - 1).bit_length()
        bound = Fraction(max(1, int(math.log2(P)))) * Fraction(1, 2 ** 24) * exact
        assert abs(Fraction(float(oracle.tree_sum(v))) - exact) <= bound


# ----------------------------------------------------------------------------
# ternarize (hand-derived examples)
# ----------------------------------------------------------------------------

def test_ternarize_threshold_equality(oracle):
    # x = [3, 1, 1, -3]: tree = (3+1)+(1+3) = 8, mu = 2, thr = 1; |1| <= 1 -> 0.
    t, alpha, nnz = oracle.ternarize(np.array([[3, 1, 1, -3]], np.float32))
    assert t.tolist() == [[1, 0, 0, -1]]
    assert nnz.tolist() == [2]
    assert alpha[0] == F(3)  # ((3+0)+(0+3)) / 2
    mask = oracle.pack_plane(t, "mask")
    sign = oracle.pack_plane(t, "sign")
    assert mask.tolist() == [[0x09, 0, 0, 0, 0, 0, 0, 0]]
    assert sign.tolist() == [[0x08, 0, 0, 0, 0, 0, 0, 0]]


def test_ternarize_non_power_of_two(oracle):
    # x = [1, 2, 4]: tree = (1+2)+(4+0) = 7, mu = fl32(7/3), thr = mu/2 ~ 1.1667.
    t, alpha, nnz = oracle.ternarize(np.array([[1, 2, 4]], np.float32))
    assert t.tolist() == [[0, 1, 1]]
    assert nnz.tolist() == [2] and alpha[0] == F(3)
    assert oracle.pack_plane(t, "mask")[0, 0] == 0x06
    assert oracle.pack_plane(t, "sign")[0, 0] == 0x00


def test_ternarize_signed_zero_and_zero_rows(oracle):
    # [-0.0, 4, -4, 0]: mu = 2, thr = 1 -> t = [0, 1, -1, 0]; alpha = 8/2 = 4.
    t, alpha, nnz = oracle.ternarize(np.array([[-0.0, 4, -4, 0], [0, 0, 0, 0], [-0.0] * 4],
                                              np.float32))
    assert t.tolist() == [[0, 1, -1, 0], [0, 0, 0, 0], [0, 0, 0, 0]]
    assert alpha.tolist() == [4.0, 0.0, 0.0] and nnz.tolist() == [2, 0, 0]
    assert oracle.pack_plane(t, "sign")[0, 0] == 0x04


def test_ternarize_padding_k65(oracle):
    # K = 65 pads to 128 bits (16 bytes).  x = [1]*64 + [2]: tree = 64 + 2 = 66,
    # mu = fl32(66/65) ~ 1.015, thr ~ 0.508 -> every value survives.
    x = np.array([[1.0] * 64 + [2.0]], np.float32)
    t, alpha, nnz = oracle.ternarize(x)
    assert (t == 1).all() and nnz[0] == 65
    assert alpha[0] == F(66) / F(65)
    mask = oracle.pack_plane(t, "mask")
    assert mask.shape == (1, 16)
    assert mask[0].tolist() == [0xFF] * 8 + [0x01] + [0] * 7


def test_ternarize_constant_row(oracle):
    # |x| = c everywhere: mu = c, thr = c/2, every value survives with alpha = c.
    for c in [0.5, 3.0, 1e-3]:
        x = np.full((1, 256), c, np.float32)
        x[0, ::3] *= -1
        t, alpha, nnz = oracle.ternarize(x)
        assert nnz[0] == 256 and alpha[0] == F(c)
        assert (t[0] == np.where(x[0] < 0, -1, 1)).all()


def test_ternarize_brute_force_small(oracle):
    # Independent scalar re-derivation with numpy float32 scalars and a recursive tree.
    def tree(v):
        P = 1
        while P < len(v):
            P *= 2
        v = list(v) + [F(0)] * (P - len(v))

        def rec(a):
            if len(a) == 1:
                return F(a[0])
            h = len(a) // 2
            return F(rec(a[:h]) + rec(a[h:]))
        return rec(v)

    rng = np.random.default_rng(5)
    for K in [1, 2, 3, 7, 31, 64, 65, 70, 129]:
        x = rng.standard_t(4, size=(3, K)).astype(np.float32)
        t, alpha, nnz = oracle.ternarize(x)
        for r in range(3):
            a = [F(abs(v)) for v in x[r]]
            mu = F(tree(a) / F(K))
            thr = F(F(0.5) * mu)
            tt = [0 if a[k] <= thr else (-1 if x[r, k] < 0 else 1) for k in range(K)]
            assert t[r].tolist() == tt
            n = sum(1 for v in tt if v)
            assert nnz[r] == n
            kept = [a[k] if tt[k] else F(0) for k in range(K)]
            assert alpha[r] == (F(tree(kept) / F(n)) if n else F(0))


def test_ternarize_invariants(oracle):
    rng = np.random.default_rng(6)
    x = rng.standard_t(3, size=(16, 300)).astype(np.float32)
    t, alpha, nnz = oracle.ternarize(x)
    # scaling by a power of two keeps t and scales alpha exactly
    for e in [-3, 5]:
        t2, a2, n2 = oracle.ternarize(x * F(2.0 ** e))
        assert (t2 == t).all() and (n2 == nnz).all() and (a2 == alpha * F(2.0 ** e)).all()
    # negation flips t, keeps alpha and nnz
    t3, a3, n3 = oracle.ternarize(-x)
    assert (t3 == -t).all() and (a3 == alpha).all() and (n3 == nnz).all()
    # survivors are exactly the entries with |x| > 0.5 * mean|x|
    mean_abs = np.abs(x.astype(np.float64)).mean(axis=1)
    for r in range(16):
        kept = t[r] != 0
        margin = np.abs(np.abs(x[r]) - 0.5 * mean_abs[r])
        safe = margin > 1e-5 * mean_abs[r]
        assert (kept[safe] == (np.abs(x[r]) > 0.5 * mean_abs[r])[safe]).all()
        # alpha is the mean of the surviving magnitudes (within fp32 tree error)
        if nnz[r]:
            ref = np.abs(x[r][kept].astype(np.float64)).mean()
            assert abs(alpha[r] - ref) <= 1e-5 * ref


def test_ternarize_rejects_nonfinite(oracle):
    with pytest.raises(ValueError):
        oracle.ternarize(np.array([[1.0, np.nan, 2.0]], np.float32))
    with pytest.raises(ValueError):
        oracle.binarize(np.array([[1.0, np.inf]], np.float32))


# ----------------------------------------------------------------------------
# binarize
# ----------------------------------------------------------------------------

def test_binarize_hand_example(oracle):
    # [0.5, -0.25, -0.0, -0.25]: sign bits at k = 1, 3 (-0.0 counts as +1) -> 0x0A;
    # alpha = ((0.5 + 0.25) + (0 + 0.25)) / 4 = 0.25.
    s, alpha = oracle.binarize(np.array([[0.5, -0.25, -0.0, -0.25]], np.float32))
    assert s.tolist() == [[1, -1, 1, -1]]
    assert alpha[0] == F(0.25)
    assert oracle.pack_plane(s, "sign")[0, 0] == 0x0A


def test_binarize_strided_matches_transpose(oracle):
    rng = np.random.default_rng(7)
    V = rng.standard_normal((130, 70)).astype(np.float32)   # [tokens, channels]
    s1, a1 = oracle.binarize(V, transpose=True)            # per channel
    s2, a2 = oracle.binarize(np.ascontiguousarray(V.T))
    assert (s1 == s2).all() and (a1 == a2).all()
    assert s1.shape == (70, 130)


def test_binarize_alpha_is_mean_abs(oracle):
    rng = np.random.default_rng(8)
    W = (rng.standard_normal((32, 1000)) * 0.02).astype(np.float32)
    s, alpha = oracle.binarize(W)
    assert (s == np.where(W < 0, -1, 1)).all()
    ref = np.abs(W.astype(np.float64)).mean(axis=1)
    assert np.all(np.abs(alpha - ref) <= 1e-5 * ref)


# ----------------------------------------------------------------------------
# packing
# ----------------------------------------------------------------------------

def test_pack_plane_matches_numpy_packbits(oracle):
    rng = np.random.default_rng(9)
    for K in [1, 8, 63, 64, 65, 100, 1000]:
        v = rng.integers(-1, 2, size=(5, K)).astype(np.int8)
        Kp = (K + 63) // 64 * 64
        for which, bits in [("mask", v != 0), ("sign", v < 0)]:
            padded = np.zeros((5, Kp), np.uint8)
            padded[:, :K] = bits
            ref = np.packbits(padded, axis=1, bitorder="little")
            assert (oracle.pack_plane(v, which) == ref).all()


def test_bits_per_value(oracle):
    # The page states one bit per weight and two per activation.
    with open(os.path.join(HERE, "golden", "bits_per_value.json")) as f:
        g = json.load(f)
    K = 4096
    rng = np.random.default_rng(10)
    x = rng.standard_t(3, size=(4, K)).astype(np.float32)
    w = rng.standard_normal((4, K)).astype(np.float32)
    t, _, _ = oracle.ternarize(x)
    s, _ = oracle.binarize(w)
    act_bytes = oracle.pack_plane(t, "mask").nbytes + oracle.pack_plane(t, "sign").nbytes
    w_bytes = oracle.pack_plane(s, "sign").nbytes
    assert w_bytes * 8 == g["weight_bits_per_value"] * 4 * K
    assert act_bytes * 8 == g["activation_bits_per_value"] * 4 * K


# ----------------------------------------------------------------------------
# integer product
# ----------------------------------------------------------------------------

def _popc(a):
    return np.unpackbits(a.view(np.uint8), axis=-1).sum(axis=-1).astype(np.int64)


def test_matmul_vs_float64_matmul(oracle):
    rng = np.random.default_rng(11)
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (17, 9, 64), (33, 40, 65), (64, 64, 200)]:
        A = rng.integers(-1, 2, size=(M, K)).astype(np.int8)
        B = rng.choice([-1, 1], size=(N, K)).astype(np.int8)
        acc = oracle.matmul_i32(A, B)
        ref = A.astype(np.float64) @ B.astype(np.float64).T   # exact below 2^53
        assert (acc == ref.astype(np.int64)).all()


def test_matmul_brute_force_triple_loop(oracle):
    rng = np.random.default_rng(12)
    A = rng.integers(-1, 2, size=(4, 11)).astype(np.int8)
    B = rng.integers(-1, 2, size=(3, 11)).astype(np.int8)
    acc = oracle.matmul_i32(A, B)
    for m in range(4):
        for n in range(3):
            assert acc[m, n] == sum(int(A[m, k]) * int(B[n, k]) for k in range(11))


def test_matmul_threads_and_pairs(oracle):
    rng = np.random.default_rng(13)
    A = rng.integers(-1, 2, size=(37, 300)).astype(np.int8)
    B = rng.choice([-1, 1], size=(23, 300)).astype(np.int8)
    a1 = oracle.matmul_i32(A, B, threads=1)
    a4 = oracle.matmul_i32(A, B, threads=4)
    assert (a1 == a4).all()
    mi = rng.integers(0, 37, size=50)
    ni = rng.integers(0, 23, size=50)
    assert (oracle.matmul_i32_pairs(A, B, mi, ni) == a1[mi, ni]).all()


def test_popcount_identities(oracle):
    """acc = popc(m & ~(w^a)) - popc(m & (w^a)) = nnz - 2 popc(bfi(w, m^a, a))."""
    rng = np.random.default_rng(14)
    M, N, K = 9, 7, 200
    x = rng.standard_t(4, size=(M, K)).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    t, _, nnz = oracle.ternarize(x)
    s, _ = oracle.binarize(w)
    acc = oracle.matmul_i32(t, s)
    m = oracle.pack_plane(t, "mask").view(np.uint64)
    a = oracle.pack_plane(t, "sign").view(np.uint64)
    ws = oracle.pack_plane(s, "sign").view(np.uint64)
    for i in range(M):
        for j in range(N):
            d = ws[j] ^ a[i]
            pos = _popc(m[i] & ~d)
            neg = _popc(m[i] & d)
            assert acc[i, j] == pos - neg
            bfi = (ws[j] & (m[i] ^ a[i])) | (~ws[j] & a[i])
            assert acc[i, j] == nnz[i] - 2 * _popc(bfi)


def test_ternary_ternary_identity(oracle):
    """Sum tq*tk = popc(mq & mk) - 2 popc(mq & mk & (aq ^ ak))."""
    rng = np.random.default_rng(15)
    q = rng.standard_normal((6, 128)).astype(np.float32)
    k = rng.standard_normal((5, 128)).astype(np.float32)
    tq, _, _ = oracle.ternarize(q)
    tk, _, _ = oracle.ternarize(k)
    acc = oracle.matmul_i32(tq, tk)
    mq, aq = oracle.pack_plane(tq, "mask").view(np.uint64), oracle.pack_plane(tq, "sign").view(np.uint64)
    mk, ak = oracle.pack_plane(tk, "mask").view(np.uint64), oracle.pack_plane(tk, "sign").view(np.uint64)
    for i in range(6):
        for j in range(5):
            both = mq[i] & mk[j]
            assert acc[i, j] == _popc(both) - 2 * _popc(both & (aq[i] ^ ak[j]))
            assert abs(acc[i, j]) <= _popc(both) and (acc[i, j] - _popc(both)) % 2 == 0


def test_matmul_invariants(oracle):
    rng = np.random.default_rng(16)
    M, N, K = 20, 30, 333
    x = rng.standard_t(3, size=(M, K)).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    t, _, nnz = oracle.ternarize(x)
    s, _ = oracle.binarize(w)
    acc = oracle.matmul_i32(t, s)
    # |acc| <= nnz and acc has the parity of nnz
    assert (np.abs(acc) <= nnz[:, None]).all()
    assert ((acc - nnz[:, None]) % 2 == 0).all()
    # all-positive weights: acc = popc(m ^ a) - popc(a) = sum t
    ones = np.ones((1, K), np.int8)
    assert (oracle.matmul_i32(t, ones)[:, 0] == t.sum(axis=1)).all()
    # a consistent permutation of k leaves acc unchanged
    p = rng.permutation(K)
    assert (oracle.matmul_i32(t[:, p], s[:, p]) == acc).all()
    # negating x negates acc
    tn, _, _ = oracle.ternarize(-x)
    assert (oracle.matmul_i32(tn, s) == -acc).all()


# ----------------------------------------------------------------------------
# epilogue and bf16
# ----------------------------------------------------------------------------

def test_epilogue_hand_example(oracle):
    # x = [3,1,1,-3] -> t = [1,0,0,-1], alpha_a = 3; w = [0.5,-0.25,-0.0,-0.25] ->
    # s = [1,-1,1,-1], alpha_w = 0.25; acc = 1 + 1 = 2; y = 2 * fl32(3 * 0.25) = 1.5.
    res = oracle.linear(np.array([[3, 1, 1, -3]], np.float32),
                        np.array([[0.5, -0.25, -0.0, -0.25]], np.float32), out="bf16")
    assert res["acc"].tolist() == [[2]]
    assert res["y"].tolist() == [[1.5]]
    assert res["y_bf16"].tolist() == [[0x3FC0]]


def test_epilogue_error_bound_and_exact_cases(oracle):
    rng = np.random.default_rng(17)
    acc = rng.integers(-5000, 5000, size=(8, 9)).astype(np.int32)
    aa = np.abs(rng.standard_normal(8)).astype(np.float32) + F(0.1)
    ab = np.abs(rng.standard_normal(9)).astype(np.float32) * F(0.02) + F(1e-3)
    y = oracle.scale(acc, aa, ab)
    exact = acc.astype(np.float64) * aa.astype(np.float64)[:, None] * ab.astype(np.float64)[None]
    # two fp32 roundings: relative error <= 2u + u^2
    u = 2.0 ** -24
    assert np.all(np.abs(y - exact) <= (2 * u + u * u) * np.abs(exact))
    # powers of two: every product is exact
    p2a = np.array([0.5, 2.0, 4.0], np.float32)
    p2b = np.array([0.25, 8.0], np.float32)
    acc2 = np.array([[1, -3], [7, 0], [-1000, 12345]], np.int32)
    assert (oracle.scale(acc2, p2a, p2b) == acc2 * p2a[:, None] * p2b[None]).all()


def test_bf16_rounding_vs_torch(oracle):
    import torch
    rng = np.random.default_rng(18)
    y = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 100,
                        np.array([1.00390625, 1.01171875, -3.5, 0.0, -0.0], np.float32)])
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (oracle.to_bf16(y) == ref).all()
    assert oracle.to_bf16(np.array([1.00390625], np.float32))[0] == 0x3F80   # tie -> even
    assert oracle.to_bf16(np.array([1.01171875], np.float32))[0] == 0x3F82   # tie -> even


def test_widen_bf16_exact(oracle):
    import torch
    rng = np.random.default_rng(19)
    bits = rng.integers(0, 0x7F80, size=1000).astype(np.uint16)   # finite positives
    bits = np.concatenate([bits, bits | 0x8000])
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert (oracle.widen(bits) == ref).all()


def test_attention_probs_vs_scipy(oracle):
    from scipy.special import softmax
    rng = np.random.default_rng(20)
    acc = rng.integers(-128, 129, size=(16, 40)).astype(np.int32)
    aq = rng.uniform(0.5, 2, size=16).astype(np.float32)
    ak = rng.uniform(0.5, 2, size=40).astype(np.float32)
    P = oracle.attention_probs(acc, aq, ak, 128)
    z = aq.astype(np.float64)[:, None] * ak.astype(np.float64)[None] * acc / math.sqrt(128)
    ref = softmax(z, axis=1)
    assert np.all(np.abs(P - ref) <= 2.0 ** -23 * ref + 1e-45)
    assert np.all(P > 0)


# ----------------------------------------------------------------------------
# Two-plane residual binarization (BiLLM page, Approach: residual, second-order
# binarization of the salient weights; here applied to whole rows).
# ----------------------------------------------------------------------------

def test_residual_hand_rows(oracle):
    """Worked by hand from the definition.
    [3, -1, 1, -3]: alpha1 = ((3+1)+(1+3))/4 = 2, r = [1, 1, -1, -1], alpha2 = 1,
    so 2*s1 + 1*s2 rebuilds the row exactly.
    [0.5, -0.25, -0.0, -0.25]: alpha1 = 0.25 (-0.0 counts as +), r = [0.25, +0.0,
    -0.25, +0.0] (-0.25 + 0.25 rounds to +0; -0.0 - 0.25 = -0.25),
    s2 = [+, +, -, +], alpha2 = ((0.25+0)+(0.25+0))/4 = 0.125."""
    W = np.array([[3, -1, 1, -3], [0.5, -0.25, -0.0, -0.25]], F)
    s1, a1, s2, a2 = oracle.binarize_residual(W)
    assert s1.tolist() == [[1, -1, 1, -1], [1, -1, 1, -1]]
    assert a1.tolist() == [2.0, 0.25]
    assert s2.tolist() == [[1, 1, -1, -1], [1, 1, -1, 1]]
    assert a2.tolist() == [1.0, 0.125]


def test_residual_constant_magnitude(oracle):
    """|w| constant along a row: the residual is zero, s2 = +1, alpha2 = 0."""
    rng = np.random.default_rng(30)
    W = (np.where(rng.random((5, 96)) < 0.5, -1.0, 1.0) * 0.375).astype(F)
    s1, a1, s2, a2 = oracle.binarize_residual(W)
    assert (s1 == np.where(W < 0, -1, 1)).all()
    assert (a1 == F(0.375)).all()
    assert (s2 == 1).all() and (a2 == 0).all()


@pytest.mark.parametrize("K", [64, 256, 4096])
def test_residual_recovers_two_plane_rows(oracle, K):
    """W = alpha1*S1 + alpha2*S2 with dyadic alpha1 > alpha2 > 0 and S2 agreeing with
    S1 on exactly half of each row: |w| takes alpha1 +- alpha2 equally often, so the
    mean of |w| is alpha1, the residual is alpha2*S2, and (with dyadic values and K
    a power of two every tree sum is exact) the planes and scales come back."""
    rng = np.random.default_rng(K)
    rows = 6
    S1 = np.where(rng.random((rows, K)) < 0.5, -1, 1).astype(np.int8)
    agree = np.zeros((rows, K), bool)
    for r in range(rows):
        agree[r, rng.permutation(K)[:K // 2]] = True
    S2 = np.where(agree, S1, -S1).astype(np.int8)
    a1 = np.array([2.0 ** -e for e in range(1, rows + 1)], F)
    a2 = a1 / 4
    W = (a1[:, None] * S1 + a2[:, None] * S2).astype(F)
    s1, b1, s2, b2 = oracle.binarize_residual(W)
    assert (s1 == S1).all() and (s2 == S2).all()
    assert (b1 == a1).all() and (b2 == a2).all()


def test_scale_residual_closed_form(oracle):
    """acc1 = 3, acc2 = -1, alpha_a = 2, alpha1 = 0.5, alpha2 = 0.25: 3*1 + (-1)*0.5."""
    y = oracle.scale_residual(np.array([[3]], np.int32), np.array([[-1]], np.int32),
                              np.array([2], F), np.array([0.5], F), np.array([0.25], F))
    assert y[0, 0] == F(2.5)


def test_residual_linear_vs_float64(oracle):
    """The two-plane product against numpy's fp64 matmul of the rebuilt weights
    alpha_a * (t @ (alpha1 s1 + alpha2 s2)^T): within three fp32 roundings."""
    rng = np.random.default_rng(31)
    X = rng.standard_t(4, size=(9, 200)).astype(F)
    W = (rng.standard_normal((13, 200)) * 0.02).astype(F)
    t, aa, _ = oracle.ternarize(X)
    s1, a1, s2, a2 = oracle.binarize_residual(W)
    y = oracle.scale_residual(oracle.matmul_i32(t, s1), oracle.matmul_i32(t, s2), aa, a1, a2)
    Wr = a1.astype(np.float64)[:, None] * s1 + a2.astype(np.float64)[:, None] * s2
    ref = aa.astype(np.float64)[:, None] * (t.astype(np.float64) @ Wr.T)
    mag = aa.astype(np.float64)[:, None] * (np.abs(t).astype(np.float64) @ np.abs(Wr).T)
    assert np.all(np.abs(y - ref) <= 4 * 2.0 ** -24 * mag + 1e-30)
