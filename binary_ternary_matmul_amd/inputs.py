"""Seeded synthetic inputs for the binary-weight x ternary-activation workloads.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic (no thresholds, scales, packing or products), so the GPU
library and the CPU oracle can both be fed from it.

The workloads are stand-ins for the BERT- and LLaMA-style linear and attention
layers that the BWTA page ("BWTA: Accurate and Efficient Binarized Transformer
by Algorithm-Hardware Co-design", Abstract) evaluates; no dataset or trained
weight is needed or used.  Every tensor has its own child stream of
``numpy.random.SeedSequence(1000 + workload_index)``, spawned in a fixed order,
so each tensor can be regenerated alone.

Float tensors come back as ``float32`` arrays; bf16 tensors come back as their
``uint16`` bit patterns (fp32 rounded to nearest even).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 1000


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def student_t(rng, shape, nu: float) -> np.ndarray:
    return rng.standard_t(nu, size=shape).astype(np.float32)


def normal(rng, shape, std: float) -> np.ndarray:
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def with_outlier_channels(x: np.ndarray, rng, count: int, factor: float):
    """Scale `count` distinct channels (columns), drawn without replacement, by `factor`."""
    K = x.shape[1]
    ch = np.sort(rng.choice(K, size=count, replace=False))
    x[:, ch] *= np.float32(factor)
    return x, ch


@dataclass
class Linear:
    """One linear layer: activations X [M, K] and weights W [N, K]."""
    name: str
    M: int
    K: int
    N: int
    x_dtype: str          # "f32" or "bf16"
    out_dtype: str        # "f32" or "bf16"
    _gen_x: object = field(repr=False, default=None)
    _gen_w: object = field(repr=False, default=None)

    def x(self) -> np.ndarray:
        return self._gen_x()

    def w(self) -> np.ndarray:
        return self._gen_w()


def _mk_x(rng_seed_seq, M, K, nu, outliers, factor, bf16):
    def gen():
        rng = np.random.Generator(np.random.PCG64(rng_seed_seq))
        x = student_t(rng, (M, K), nu)
        if outliers:
            x, _ = with_outlier_channels(x, rng, outliers, factor)
        return f32_to_bf16_bits(x) if bf16 else x
    return gen


def _mk_w(rng_seed_seq, N, K, std):
    def gen():
        rng = np.random.Generator(np.random.PCG64(rng_seed_seq))
        return normal(rng, (N, K), std)
    return gen


def single_linear() -> list[Linear]:
    """Single fp32 linear: X[128, 768] Student-t(nu=4); W[768, 768] ~ N(0, 0.02)."""
    ss = np.random.SeedSequence(SEED_BASE + 0).spawn(2)
    return [Linear("linear", 128, 768, 768, "f32", "f32",
                   _mk_x(ss[0], 128, 768, 4.0, 0, 1.0, False), _mk_w(ss[1], 768, 768, 0.02))]


BERT_SHAPES = [("qkv", 768, 2304), ("out", 768, 768), ("ffn_up", 768, 3072),
               ("ffn_down", 3072, 768)]


def bert_encoder(M: int = 4096) -> list[Linear]:
    """BERT-base encoder linears, M = 32 x 128 tokens, fp32 inputs, bf16 outputs.

    X ~ Student-t(nu=4) with 8 outlier channels x20 (one X per layer); W ~ N(0, 0.02).
    """
    ss = np.random.SeedSequence(SEED_BASE + 1).spawn(2 * len(BERT_SHAPES))
    out = []
    for i, (name, K, N) in enumerate(BERT_SHAPES):
        out.append(Linear(name, M, K, N, "f32", "bf16",
                          _mk_x(ss[2 * i], M, K, 4.0, 8, 20.0, False),
                          _mk_w(ss[2 * i + 1], N, K, 0.02)))
    return out


LLAMA7B_SHAPES = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                  ("gate", 4096, 11008), ("up", 4096, 11008), ("down", 11008, 4096)]
# which activation feeds each projection: q/k/v share the attention input, gate/up
# share the MLP input; o and down have their own.
LLAMA7B_INPUTS = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "attn_out",
                  "gate": "mlp_in", "up": "mlp_in", "down": "mlp_act",
                  "qkv": "attn_in", "gate_up": "mlp_in"}


def llama7b_prefill(M: int = 2048, out_dtype: str = "bf16") -> tuple[dict, list[Linear]]:
    """LLaMA-7B-shaped prefill linears, M = 2048 tokens.

    Activations bf16 Student-t(nu=3) with round(0.01 K) outlier channels x50;
    weights N(0, 0.02).  Returns (activation generators by name, linears).
    """
    ss = np.random.SeedSequence(SEED_BASE + 2).spawn(4 + len(LLAMA7B_SHAPES))
    acts = {}
    for i, (name, K) in enumerate([("attn_in", 4096), ("attn_out", 4096), ("mlp_in", 4096),
                                   ("mlp_act", 11008)]):
        acts[name] = _mk_x(ss[i], M, K, 3.0, int(round(0.01 * K)), 50.0, True)
    lins = []
    for j, (name, K, N) in enumerate(LLAMA7B_SHAPES):
        lins.append(Linear(name, M, K, N, "bf16", out_dtype, acts[LLAMA7B_INPUTS[name]],
                           _mk_w(ss[4 + j], N, K, 0.02)))
    return acts, lins


# The seven linears as the four products a layer runs: projections that read the
# same activation have their weights stacked along N (q/k/v into [12288, 4096],
# gate/up into [22016, 4096]).  Every weight row keeps its own plane row and
# scale, so a stacked product equals its linears side by side.
LLAMA7B_PRODUCTS = [("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")),
                    ("down", ("down",))]


def stacked(name: str, lins: list[Linear]) -> Linear:
    """One Linear whose weights are those of `lins` (same activation) stacked along N."""
    first = lins[0]
    gens = [lin._gen_w for lin in lins]
    return Linear(name, first.M, first.K, sum(lin.N for lin in lins), first.x_dtype,
                  first.out_dtype, first._gen_x, lambda: np.concatenate([g() for g in gens]))


def llama7b_products(M: int = 2048, out_dtype: str = "bf16") -> tuple[dict, list[Linear]]:
    """The LLaMA-7B prefill linears as the four stacked products (LLAMA7B_PRODUCTS)."""
    acts, lins = llama7b_prefill(M, out_dtype)
    by = {lin.name: lin for lin in lins}
    return acts, [stacked(name, [by[p] for p in parts]) for name, parts in LLAMA7B_PRODUCTS]


LLAMA70B_DECODE_SHAPES = [("gate_up", 8192, 28672), ("down", 28672, 8192)]


def llama70b_decode(M: int = 1) -> list[Linear]:
    """LLaMA2-70B-shaped decode GEMV / skinny GEMM, M in {1, 4, 16}.

    x bf16 Student-t(nu=3) (the first M rows of one [16, K] draw, so the three M
    values share rows); W ~ N(0, 0.015); fp32 outputs.
    """
    assert 1 <= M <= 16
    ss = np.random.SeedSequence(SEED_BASE + 3).spawn(2 * len(LLAMA70B_DECODE_SHAPES))
    out = []
    for i, (name, K, N) in enumerate(LLAMA70B_DECODE_SHAPES):
        full = _mk_x(ss[2 * i], 16, K, 3.0, 0, 1.0, True)
        out.append(Linear(name, M, K, N, "bf16", "f32",
                          (lambda f=full, m=M: np.ascontiguousarray(f()[:m])),
                          _mk_w(ss[2 * i + 1], N, K, 0.015)))
    return out


def llama70b_up_weight():
    """The up projection of the same LLaMA2-70B MLP: W [28672, 8192] ~ N(0, 0.015), its
    own draw (the child after the decode shapes' children of the same seed).  Stacked
    under the gate weight it gives the [57344, 8192] gate/up matrix one decode launch
    reads."""
    ss = np.random.SeedSequence(SEED_BASE + 3).spawn(2 * len(LLAMA70B_DECODE_SHAPES) + 1)
    name, K, N = LLAMA70B_DECODE_SHAPES[0]
    return _mk_w(ss[-1], N, K, 0.015)


@dataclass
class Attention:
    heads: int
    L: int
    d: int
    q: np.ndarray       # [heads, L, d] bf16 bits
    k: np.ndarray
    v: np.ndarray
    scales: np.ndarray  # [3, heads] fp32 per-(tensor, head) scale


def attention(heads: int = 32, L: int = 2048, d: int = 128) -> Attention:
    """Batched attention inputs: Q, K, V bf16 ~ N(0, 1) times a per-(tensor, head)
    scale drawn from U(0.5, 2)."""
    ss = np.random.SeedSequence(SEED_BASE + 4).spawn(4)
    srng = np.random.Generator(np.random.PCG64(ss[3]))
    scales = srng.uniform(0.5, 2.0, size=(3, heads)).astype(np.float32)
    t = []
    for i in range(3):
        rng = np.random.Generator(np.random.PCG64(ss[i]))
        x = rng.standard_normal(size=(heads, L, d), dtype=np.float32)
        x *= scales[i][:, None, None]
        t.append(f32_to_bf16_bits(x))
    return Attention(heads, L, d, t[0], t[1], t[2], scales)


def random_linear(seed: int, M: int, K: int, N: int, nu: float = 4.0, std: float = 0.02,
                  bf16: bool = False):
    """Small seeded case for parity tests at arbitrary (ragged) shapes."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = student_t(rng, (M, K), nu)
    w = normal(rng, (N, K), std)
    return (f32_to_bf16_bits(x) if bf16 else x), w
