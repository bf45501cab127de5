"""ctypes binding for the scalar CPU oracle in ``bwta_oracle.c``.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; the GPU library never imports it.
It imports nothing from the GPU package either.

Every function works on host numpy arrays.  The arithmetic is in the C file;
this module only marshals arguments.  The definitions it implements are stated
at the top of ``bwta_oracle.c`` and follow "BWTA: Accurate and Efficient
Binarized Transformer by Algorithm-Hardware Co-design", Abstract (binary
weights, ternary activations with tiny values projected to zero, bit-packed
binary/ternary MatMul for linear and attention operators).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bwta_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm", "-lpthread"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_tree_sum.restype = ctypes.c_float
        lib.oracle_tree_sum.argtypes = [P, I64]
        lib.oracle_padded_k.restype = I64
        lib.oracle_padded_k.argtypes = [I64]
        lib.oracle_row_bytes.restype = I64
        lib.oracle_row_bytes.argtypes = [I64]
        lib.oracle_bf16_to_f32.argtypes = [P, P, I64]
        lib.oracle_f32_to_bf16.argtypes = [P, P, I64]
        lib.oracle_binarize.restype = ctypes.c_int
        lib.oracle_binarize.argtypes = [P, I64, I64, I64, I64, P, P]
        lib.oracle_ternarize.restype = ctypes.c_int
        lib.oracle_ternarize.argtypes = [P, I64, I64, I64, P, P, P]
        lib.oracle_pack_plane.restype = ctypes.c_int
        lib.oracle_pack_plane.argtypes = [P, I64, I64, ctypes.c_int, P]
        lib.oracle_matmul_i32.restype = ctypes.c_int
        lib.oracle_matmul_i32.argtypes = [P, P, I64, I64, I64, P, ctypes.c_int]
        lib.oracle_matmul_i32_pairs.restype = ctypes.c_int
        lib.oracle_matmul_i32_pairs.argtypes = [P, P, I64, P, P, I64, P]
        lib.oracle_scale.argtypes = [P, P, P, I64, I64, P]
        lib.oracle_binarize_residual.restype = ctypes.c_int
        lib.oracle_binarize_residual.argtypes = [P, I64, I64, I64, I64, P, P, P, P]
        lib.oracle_scale_residual.argtypes = [P, P, P, P, P, I64, I64, P]
        lib.oracle_attention_probs.argtypes = [P, P, P, I64, I64, I64, P]
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str):
    if rc == 1:
        raise ValueError(f"{what}: non-finite input (outside the contract)")
    if rc != 0:
        raise ValueError(f"{what}: bad arguments (status {rc})")


def padded_k(K: int) -> int:
    return int(_load().oracle_padded_k(K))


def row_bytes(K: int) -> int:
    return int(_load().oracle_row_bytes(K))


def tree_sum(v) -> np.float32:
    """Perfect pairwise fp32 tree over v zero-padded to a power of two."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    return np.float32(_load().oracle_tree_sum(_ptr(v), v.size))


def widen(x: np.ndarray) -> np.ndarray:
    """Return fp32 values: fp32 stays, bf16 bit patterns (uint16) widen exactly."""
    if x.dtype == np.float32:
        return np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = np.ascontiguousarray(x)
        out = np.empty(x.shape, np.float32)
        _load().oracle_bf16_to_f32(_ptr(x), _ptr(out), x.size)
        return out
    raise TypeError(f"unsupported input dtype {x.dtype}")


def to_bf16(y: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint16)
    _load().oracle_f32_to_bf16(_ptr(y), _ptr(out), y.size)
    return out


def binarize(W: np.ndarray, transpose: bool = False):
    """Binary weights of the rows of W (or of its columns when transpose=True).

    Returns (s, alpha): s int8 in {-1,+1} shape [rows, K]; alpha fp32 [rows].
    """
    W = widen(W)
    assert W.ndim == 2
    if transpose:
        K, rows = W.shape
        sr, sk = 1, rows
    else:
        rows, K = W.shape
        sr, sk = K, 1
    s = np.empty((rows, K), np.int8)
    alpha = np.empty(rows, np.float32)
    _check(_load().oracle_binarize(_ptr(W), rows, K, sr, sk, _ptr(s), _ptr(alpha)), "binarize")
    return s, alpha


def binarize_residual(W: np.ndarray):
    """Two binary planes per row of W (BiLLM page, Approach: residual binarization):
    (s1, alpha1) = binarize(W), then (s2, alpha2) = binarize of the residual
    r = W - alpha1 * s1 in fp32.  Returns (s1, alpha1, s2, alpha2)."""
    W = widen(W)
    assert W.ndim == 2
    rows, K = W.shape
    s1 = np.empty((rows, K), np.int8)
    s2 = np.empty((rows, K), np.int8)
    a1 = np.empty(rows, np.float32)
    a2 = np.empty(rows, np.float32)
    _check(_load().oracle_binarize_residual(_ptr(W), rows, K, K, 1, _ptr(s1), _ptr(a1), _ptr(s2),
                                            _ptr(a2)), "binarize_residual")
    return s1, a1, s2, a2


def ternarize(X: np.ndarray):
    """Ternary activations of the rows of X.

    Returns (t, alpha, nnz): t int8 in {-1,0,+1} [rows, K]; alpha fp32 [rows];
    nnz int32 [rows].
    """
    X = widen(X)
    assert X.ndim == 2
    rows, K = X.shape
    t = np.empty((rows, K), np.int8)
    alpha = np.empty(rows, np.float32)
    nnz = np.empty(rows, np.int32)
    _check(_load().oracle_ternarize(_ptr(X), rows, K, K, _ptr(t), _ptr(alpha), _ptr(nnz)),
           "ternarize")
    return t, alpha, nnz


def pack_plane(v: np.ndarray, which: str) -> np.ndarray:
    """Bit plane of int8 values: which='mask' -> (v != 0), 'sign' -> (v < 0).

    Returns uint8 [rows, row_bytes(K)]; byte b bit j (LSB first) holds k = 8b + j.
    """
    v = np.ascontiguousarray(v, dtype=np.int8)
    rows, K = v.shape
    out = np.empty((rows, row_bytes(K)), np.uint8)
    _check(_load().oracle_pack_plane(_ptr(v), rows, K, 0 if which == "mask" else 1, _ptr(out)),
           "pack_plane")
    return out


def matmul_i32(A: np.ndarray, B: np.ndarray, threads: int = 1) -> np.ndarray:
    """acc[m, n] = sum_k A[m, k] * B[n, k] in int32 over unpacked int8 values."""
    A = np.ascontiguousarray(A, dtype=np.int8)
    B = np.ascontiguousarray(B, dtype=np.int8)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    _check(_load().oracle_matmul_i32(_ptr(A), _ptr(B), M, N, K, _ptr(acc), int(threads)),
           "matmul")
    return acc


def matmul_i32_pairs(A: np.ndarray, B: np.ndarray, mi, ni) -> np.ndarray:
    """acc[mi[i], ni[i]] for a list of index pairs."""
    A = np.ascontiguousarray(A, dtype=np.int8)
    B = np.ascontiguousarray(B, dtype=np.int8)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    assert A.shape[1] == B.shape[1] and mi.shape == ni.shape
    assert (mi >= 0).all() and (mi < A.shape[0]).all() and (ni >= 0).all() and (ni < B.shape[0]).all()
    out = np.empty(mi.shape, np.int32)
    _check(_load().oracle_matmul_i32_pairs(_ptr(A), _ptr(B), A.shape[1], _ptr(mi), _ptr(ni),
                                           mi.size, _ptr(out)), "matmul_pairs")
    return out


def scale(acc: np.ndarray, alpha_a: np.ndarray, alpha_b: np.ndarray) -> np.ndarray:
    """y[m, n] = fl32((float)acc * fl32(alpha_a[m] * alpha_b[n]))."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    alpha_a = np.ascontiguousarray(alpha_a, dtype=np.float32)
    alpha_b = np.ascontiguousarray(alpha_b, dtype=np.float32)
    M, N = acc.shape
    assert alpha_a.shape == (M,) and alpha_b.shape == (N,)
    y = np.empty((M, N), np.float32)
    _load().oracle_scale(_ptr(acc), _ptr(alpha_a), _ptr(alpha_b), M, N, _ptr(y))
    return y


def scale_residual(acc1: np.ndarray, acc2: np.ndarray, alpha_a: np.ndarray,
                   alpha1: np.ndarray, alpha2: np.ndarray) -> np.ndarray:
    """y = fl32(fl32(acc1 * fl32(alpha_a * alpha1)) + fl32(acc2 * fl32(alpha_a * alpha2)))."""
    acc1 = np.ascontiguousarray(acc1, dtype=np.int32)
    acc2 = np.ascontiguousarray(acc2, dtype=np.int32)
    alpha_a = np.ascontiguousarray(alpha_a, dtype=np.float32)
    alpha1 = np.ascontiguousarray(alpha1, dtype=np.float32)
    alpha2 = np.ascontiguousarray(alpha2, dtype=np.float32)
    M, N = acc1.shape
    assert acc2.shape == (M, N) and alpha_a.shape == (M,)
    assert alpha1.shape == (N,) and alpha2.shape == (N,)
    y = np.empty((M, N), np.float32)
    _load().oracle_scale_residual(_ptr(acc1), _ptr(acc2), _ptr(alpha_a), _ptr(alpha1),
                                  _ptr(alpha2), M, N, _ptr(y))
    return y


def attention_probs(acc: np.ndarray, alpha_q: np.ndarray, alpha_k: np.ndarray,
                    head_dim: int) -> np.ndarray:
    """Row softmax (fp64, rounded to fp32) of alpha_q*alpha_k*acc/sqrt(head_dim)."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    alpha_q = np.ascontiguousarray(alpha_q, dtype=np.float32)
    alpha_k = np.ascontiguousarray(alpha_k, dtype=np.float32)
    M, N = acc.shape
    P = np.empty((M, N), np.float32)
    _load().oracle_attention_probs(_ptr(acc), _ptr(alpha_q), _ptr(alpha_k), M, N, head_dim,
                                   _ptr(P))
    return P


# ---------------------------------------------------------------------------
# Composite helpers: the whole linear path, from float inputs to outputs.
# ---------------------------------------------------------------------------

def linear(X: np.ndarray, W: np.ndarray, out: str = "f32", threads: int = 1) -> dict:
    """Ternarize X, binarize W, multiply, rescale.  Returns every intermediate."""
    t, a_alpha, nnz = ternarize(X)
    s, w_alpha = binarize(W)
    acc = matmul_i32(t, s, threads=threads)
    y = scale(acc, a_alpha, w_alpha)
    res = dict(t=t, a_alpha=a_alpha, nnz=nnz, a_mask=pack_plane(t, "mask"),
               a_sign=pack_plane(t, "sign"), s=s, w_alpha=w_alpha, w_sign=pack_plane(s, "sign"),
               acc=acc, y=y)
    if out == "bf16":
        res["y_bf16"] = to_bf16(y)
    return res
