"""Thin ctypes binding of libbwta.so.

Only argument marshalling lives here: tensors are checked for device, dtype
and contiguity, outputs are allocated with torch (device memory is torch's
job), and every operation runs in the library's HIP kernels on the current
torch stream.  The library must be built (``python -m
binary_ternary_matmul_amd.build``); if it is missing every call raises.

The names match the C entry points declared in include/bwta.h.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import torch  # loads torch's HIP runtime first, so libbwta binds to the same one

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbwta.so")

BWTA_OK, BWTA_ERR_INVALID, BWTA_ERR_ALIGN, BWTA_ERR_UNSUPPORTED, BWTA_ERR_HIP = range(5)
DTYPES = {"f32": 0, "bf16": 1, "i32": 2}
ALGOS = {"auto": 0, "mfma": 1, "popcount": 2, "mfma_i8": 3}
_TORCH_DT = {torch.float32: 0, torch.bfloat16: 1, torch.int32: 2}
_OUT_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}

_lib = None


class BwtaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libbwta.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m binary_ternary_matmul_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.bwta_version.restype = I32
    L.bwta_padded_k.restype = I64
    L.bwta_padded_k.argtypes = [I64]
    L.bwta_row_bytes.restype = I64
    L.bwta_row_bytes.argtypes = [I64]
    L.bwta_status_string.restype = ctypes.c_char_p
    L.bwta_status_string.argtypes = [I32]
    L.bwta_last_error.restype = ctypes.c_char_p
    L.bwta_pack_weights.restype = I32
    L.bwta_pack_weights.argtypes = [P, I32, I64, I64, I64, I64, P, P, P]
    L.bwta_ternarize_pack.restype = I32
    L.bwta_ternarize_pack.argtypes = [P, I32, I64, I64, I64, P, P, P, P, P]
    prod = [P, P, P, P, P, P, I64, I64, I64, P, I32, I64, I32, P]
    L.bwta_gemm.restype = I32
    L.bwta_gemm.argtypes = prod
    L.bwta_gemv.restype = I32
    L.bwta_gemv.argtypes = prod
    L.bwta_batched_gemm.restype = I32
    L.bwta_batched_gemm.argtypes = [I64, P, P, P, P, I64, P, P, P, I64, I64, I64, I64, P, I32,
                                    I64, I64, I32, P]
    L.bwta_pack_weights_residual.restype = I32
    L.bwta_pack_weights_residual.argtypes = [P, I32, I64, I64, I64, P, P, P]
    L.bwta_gemm_residual.restype = I32
    L.bwta_gemm_residual.argtypes = [P, P, P, P, P, P, I64, I64, I64, P, I32, I64, P]
    L.bwta_gemv_residual.restype = I32
    L.bwta_gemv_residual.argtypes = [P, P, P, P, P, P, I64, I64, I64, P, I32, I64, P]
    L.bwta_attention.restype = I32
    L.bwta_attention.argtypes = [I64, I64, I64, P, P, P, P, P, P, P, P, ctypes.c_float, P, I32,
                                 P, P, P, P, P]
    _lib = L
    return L


def _check(status: int, what: str):
    if status != BWTA_OK:
        msg = lib().bwta_last_error().decode(errors="replace")
        name = lib().bwta_status_string(status).decode()
        raise BwtaError(status, f"{what}: {name}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def padded_k(K: int) -> int:
    return int(lib().bwta_padded_k(K))


def row_bytes(K: int) -> int:
    return int(lib().bwta_row_bytes(K))


class TernaryPlanes(NamedTuple):
    """Ternary matrix [rows, K]: mask/sign planes [rows, row_bytes(K)] uint8,
    alpha [rows] fp32, nnz [rows] int32."""
    mask: torch.Tensor
    sign: torch.Tensor
    alpha: torch.Tensor
    nnz: torch.Tensor
    K: int


class BinaryPlanes(NamedTuple):
    """Binary matrix [rows, K]: sign plane [rows, row_bytes(K)] uint8, alpha [rows] fp32."""
    sign: torch.Tensor
    alpha: torch.Tensor
    K: int


def _dev_check(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def bwta_pack_weights(W: torch.Tensor, transpose: bool = False) -> BinaryPlanes:
    """Binarize the rows of W [rows, K] (or its columns when transpose=True:
    W is then [K, rows] and column c becomes row c of the planes)."""
    _dev_check(W, "W")
    if W.dtype not in (torch.float32, torch.bfloat16) or W.dim() != 2:
        raise ValueError("W must be a 2-D float32 or bfloat16 tensor")
    if transpose:
        K, rows = W.shape
        sr, sk = W.stride(1), W.stride(0)
    else:
        rows, K = W.shape
        sr, sk = W.stride(0), W.stride(1)
    sign = torch.empty((rows, row_bytes(K)), dtype=torch.uint8, device=W.device)
    alpha = torch.empty(rows, dtype=torch.float32, device=W.device)
    _check(lib().bwta_pack_weights(_ptr(W), _TORCH_DT[W.dtype], rows, K, sr, sk, _ptr(sign),
                                   _ptr(alpha), _stream()), "bwta_pack_weights")
    return BinaryPlanes(sign, alpha, K)


def bwta_ternarize_pack(X: torch.Tensor) -> TernaryPlanes:
    """Ternarize the rows of X [rows, K] (unit stride along K)."""
    _dev_check(X, "X")
    if X.dtype not in (torch.float32, torch.bfloat16) or X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D float32/bfloat16 tensor with unit stride along K")
    rows, K = X.shape
    rb = row_bytes(K)
    mask = torch.empty((rows, rb), dtype=torch.uint8, device=X.device)
    sign = torch.empty((rows, rb), dtype=torch.uint8, device=X.device)
    alpha = torch.empty(rows, dtype=torch.float32, device=X.device)
    nnz = torch.empty(rows, dtype=torch.int32, device=X.device)
    _check(lib().bwta_ternarize_pack(_ptr(X), _TORCH_DT[X.dtype], rows, K, X.stride(0), _ptr(mask),
                                     _ptr(sign), _ptr(alpha), _ptr(nnz), _stream()),
           "bwta_ternarize_pack")
    return TernaryPlanes(mask, sign, alpha, nnz, K)


def _product(fn, name, a: TernaryPlanes, w: BinaryPlanes, out_dtype: str, algo: str,
             out: Optional[torch.Tensor]):
    if a.K != w.K:
        raise ValueError(f"K mismatch: activations {a.K}, weights {w.K}")
    M, N = a.mask.shape[0], w.sign.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=_OUT_TORCH[out_dtype], device=a.mask.device)
    if out.dim() != 2 or out.shape[0] != M or out.shape[1] < N or out.stride(1) != 1:
        raise ValueError("out must be [M, >=N] with unit column stride")
    _check(fn(_ptr(a.mask), _ptr(a.sign), _ptr(a.alpha), _ptr(a.nnz), _ptr(w.sign), _ptr(w.alpha),
              M, N, a.K, _ptr(out), DTYPES[out_dtype], out.stride(0), ALGOS[algo], _stream()), name)
    return out


def bwta_gemm(a: TernaryPlanes, w: BinaryPlanes, out_dtype: str = "f32", algo: str = "auto",
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y[M, N] = alpha_a * alpha_w * (t @ s^T) for the prefill linear."""
    return _product(lib().bwta_gemm, "bwta_gemm", a, w, out_dtype, algo, out)


def bwta_gemv(a: TernaryPlanes, w: BinaryPlanes, out_dtype: str = "f32", algo: str = "auto",
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode product for M <= 16 activation rows."""
    return _product(lib().bwta_gemv, "bwta_gemv", a, w, out_dtype, algo, out)


def bwta_batched_gemm(batch: int, a: TernaryPlanes, a_batch_rows: int, b, b_batch_rows: int,
                      M: int, N: int, out_dtype: str = "f32", algo: str = "auto",
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Batched products for attention: B ternary (TernaryPlanes, e.g. Q K^T) or
    binary (BinaryPlanes, e.g. P V with V^T packed per channel).
    Returns Y [batch, M, N]."""
    K = a.K
    if b.K != K:
        raise ValueError("K mismatch")
    b_mask = b.mask if isinstance(b, TernaryPlanes) else None
    if out is None:
        out = torch.empty((batch, M, N), dtype=_OUT_TORCH[out_dtype], device=a.mask.device)
    if out.dim() != 3 or out.stride(2) != 1 or tuple(out.shape) != (batch, M, N):
        raise ValueError("out must be [batch, M, N] with unit column stride")
    _check(lib().bwta_batched_gemm(batch, _ptr(a.mask), _ptr(a.sign), _ptr(a.alpha), _ptr(a.nnz),
                                   a_batch_rows, _ptr(b_mask), _ptr(b.sign), _ptr(b.alpha),
                                   b_batch_rows, M, N, K, _ptr(out), DTYPES[out_dtype],
                                   out.stride(1), out.stride(0), ALGOS[algo], _stream()),
           "bwta_batched_gemm")
    return out


class AttentionProbs(NamedTuple):
    """P of a fused attention call and its ternarization: p [heads * L, L] fp32,
    mask [heads * L, row_bytes(L)] uint8, alpha [heads * L] fp32, nnz int32."""
    p: torch.Tensor
    mask: torch.Tensor
    alpha: torch.Tensor
    nnz: torch.Tensor


def bwta_attention(q: TernaryPlanes, k: TernaryPlanes, v: BinaryPlanes, heads: int,
                   scale: Optional[float] = None, out_dtype: str = "f32",
                   out: Optional[torch.Tensor] = None, probs: bool = False):
    """Fused attention: Q, K ternary [heads * L, D] planes, v = V^T binary planes
    [heads * D, L] (bwta_pack_weights(V [L, heads * D], transpose=True)).
    scale defaults to 1 / sqrt(D).  Returns O [heads, L, D], and with probs=True
    also the AttentionProbs the kernel computed on the way."""
    D = q.K
    rows = q.mask.shape[0]
    if heads <= 0 or rows % heads:
        raise ValueError("q rows must be heads * L")
    L = rows // heads
    if k.K != D or k.mask.shape[0] != rows:
        raise ValueError("k must match q: [heads * L, D]")
    if v.K != L or v.sign.shape[0] != heads * D:
        raise ValueError("v must be V^T planes [heads * D, L]")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    dev = q.mask.device
    if out is None:
        out = torch.empty((heads, L, D), dtype=_OUT_TORCH[out_dtype], device=dev)
    if tuple(out.shape) != (heads, L, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [heads, L, D] tensor")
    pr = None
    if probs:
        pr = AttentionProbs(torch.empty((rows, L), dtype=torch.float32, device=dev),
                            torch.empty((rows, row_bytes(L)), dtype=torch.uint8, device=dev),
                            torch.empty(rows, dtype=torch.float32, device=dev),
                            torch.empty(rows, dtype=torch.int32, device=dev))
    _check(lib().bwta_attention(heads, L, D, _ptr(q.mask), _ptr(q.sign), _ptr(q.alpha),
                                _ptr(k.mask), _ptr(k.sign), _ptr(k.alpha), _ptr(v.sign),
                                _ptr(v.alpha), ctypes.c_float(scale), _ptr(out),
                                DTYPES[out_dtype], _ptr(pr.p if pr else None),
                                _ptr(pr.mask if pr else None), _ptr(pr.alpha if pr else None),
                                _ptr(pr.nnz if pr else None), _stream()), "bwta_attention")
    return (out, pr) if probs else out


class ResidualPlanes(NamedTuple):
    """Two-plane residual binary weights of N rows: sign [2N, row_bytes(K)] uint8
    and alpha [2N] fp32, interleaved in groups of 32 rows (plane 1 of rows
    32p..32p+31, then plane 2 of the same rows)."""
    sign: torch.Tensor
    alpha: torch.Tensor
    K: int


def bwta_pack_weights_residual(W: torch.Tensor) -> ResidualPlanes:
    """Two binary planes per row of W [N, K] (N a multiple of 32)."""
    _dev_check(W, "W")
    if W.dtype not in (torch.float32, torch.bfloat16) or W.dim() != 2 or W.stride(1) != 1:
        raise ValueError("W must be a 2-D float32/bfloat16 tensor with unit stride along K")
    rows, K = W.shape
    sign = torch.empty((2 * rows, row_bytes(K)), dtype=torch.uint8, device=W.device)
    alpha = torch.empty(2 * rows, dtype=torch.float32, device=W.device)
    _check(lib().bwta_pack_weights_residual(_ptr(W), _TORCH_DT[W.dtype], rows, K, W.stride(0),
                                            _ptr(sign), _ptr(alpha), _stream()),
           "bwta_pack_weights_residual")
    return ResidualPlanes(sign, alpha, K)


def bwta_gemm_residual(a: TernaryPlanes, w: ResidualPlanes, out_dtype: str = "f32",
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y[M, N] = alpha_a * (alpha1 * (t @ s1^T) + alpha2 * (t @ s2^T))."""
    return _residual(lib().bwta_gemm_residual, "bwta_gemm_residual", a, w, out_dtype, out)


def bwta_gemv_residual(a: TernaryPlanes, w: ResidualPlanes, out_dtype: str = "f32",
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The same product for M <= 16 activation rows (decode)."""
    return _residual(lib().bwta_gemv_residual, "bwta_gemv_residual", a, w, out_dtype, out)


def _residual(fn, name, a: TernaryPlanes, w: ResidualPlanes, out_dtype: str,
              out: Optional[torch.Tensor]) -> torch.Tensor:
    if a.K != w.K:
        raise ValueError(f"K mismatch: activations {a.K}, weights {w.K}")
    M, N = a.mask.shape[0], w.sign.shape[0] // 2
    if out is None:
        out = torch.empty((M, N), dtype=_OUT_TORCH[out_dtype], device=a.mask.device)
    if out.dim() != 2 or out.shape[0] != M or out.shape[1] < N or out.stride(1) != 1:
        raise ValueError("out must be [M, >=N] with unit column stride")
    _check(fn(_ptr(a.mask), _ptr(a.sign), _ptr(a.alpha), _ptr(a.nnz), _ptr(w.sign),
              _ptr(w.alpha), M, N, a.K, _ptr(out), DTYPES[out_dtype], out.stride(0), _stream()),
           name)
    return out
