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
    SZ = ctypes.c_size_t
    prod = [P, P, P, P, P, P, I64, I64, I64, P, I32, I64, I32, P, SZ, P]
    L.bwta_gemm.restype = I32
    L.bwta_gemm.argtypes = prod
    L.bwta_gemv.restype = I32
    L.bwta_gemv.argtypes = prod
    L.bwta_gemv_fused.restype = I32
    L.bwta_gemv_fused.argtypes = [P, I32, I64, P, P, I64, I64, I64, P, I32, I64, P, P, P, P, P,
                                  SZ, P]
    L.bwta_gemv_noalloc.restype = I32
    L.bwta_gemv_noalloc.argtypes = [P, P, P, P, P, P, I64, I64, I64, P, I32, I64, I32, P]
    for f in (L.bwta_gemm_workspace_size, L.bwta_gemv_workspace_size):
        f.restype = SZ
        f.argtypes = [I64, I64, I64, I32]
    L.bwta_gemv_fused_workspace_size.restype = SZ
    L.bwta_gemv_fused_workspace_size.argtypes = [I64, I64, I64]
    L.bwta_set_fused_spin_limit.restype = None
    L.bwta_set_fused_spin_limit.argtypes = [I32]
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


def _check_vec(t: Optional[torch.Tensor], n: int, dtype, name: str):
    """A contiguous 1-D tensor of n elements of `dtype`."""
    if t is None:
        raise ValueError(f"{name} is missing")
    if t.dtype != dtype or t.dim() != 1 or t.shape[0] != n or (n > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous [{n}] {dtype} tensor "
                         f"(got {tuple(t.shape)} {t.dtype})")


def _check_plane(t: torch.Tensor, rows: int, K: int, name: str):
    """A packed plane: uint8 [rows, row_bytes(K)] with rows packed back to back."""
    rb = row_bytes(K)
    if t.dtype != torch.uint8 or t.dim() != 2 or tuple(t.shape) != (rows, rb):
        raise ValueError(f"{name} must be a uint8 [{rows}, {rb}] plane "
                         f"(got {tuple(t.shape)} {t.dtype})")
    if rows > 0 and (t.stride(1) != 1 or (rows > 1 and t.stride(0) != rb)):
        raise ValueError(f"{name} must have strides ({rb}, 1) (got {t.stride()})")


def _check_ternary(a: "TernaryPlanes", name: str) -> int:
    """Check a ternary operand's planes, alpha and nnz; return its row count."""
    rows = a.mask.shape[0] if a.mask.dim() == 2 else -1
    _check_plane(a.mask, rows, a.K, f"{name}.mask")
    _check_plane(a.sign, rows, a.K, f"{name}.sign")
    _check_vec(a.alpha, rows, torch.float32, f"{name}.alpha")
    _check_vec(a.nnz, rows, torch.int32, f"{name}.nnz")
    return rows


def _check_binary(w, rows_per_alpha: int, name: str) -> int:
    """Check a binary operand (sign plane and alpha); return its plane row count."""
    rows = w.sign.shape[0] if w.sign.dim() == 2 else -1
    _check_plane(w.sign, rows, w.K, f"{name}.sign")
    _check_vec(w.alpha, rows * rows_per_alpha, torch.float32, f"{name}.alpha")
    return rows


def _check_out(out: torch.Tensor, out_dtype: str, shape, device, name: str = "out"):
    """The output: dtype `out_dtype`, `shape` (the last dimension may be a
    prefix of a wider row), unit stride along its rows, on `device`."""
    want = _OUT_TORCH[out_dtype]
    if out.dtype != want:
        raise ValueError(f"{name} has dtype {out.dtype} but out_dtype={out_dtype!r} "
                         f"writes {want}")
    if out.dim() != len(shape) or tuple(out.shape[:-1]) != tuple(shape[:-1]) or \
            out.shape[-1] < shape[-1] or out.stride(-1) != 1:
        raise ValueError(f"{name} must be {list(shape[:-1])} x >= {shape[-1]} with unit "
                         f"stride along its rows (got {tuple(out.shape)}, {out.stride()})")
    if out.device != device:
        raise ValueError(f"{name} is on {out.device}, the operands on {device}")


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


_WORKSPACE = {}  # device index -> zero-filled uint8 tensor (the "auto" workspaces)
_RETIRED = []    # workspaces replaced by larger ones: captured graphs may still use them


def workspace(device, nbytes: int) -> torch.Tensor:
    """A zero-filled workspace of at least nbytes on `device`, shared by every
    call that asks for "auto" (the library leaves its counters zero after each
    call, so one buffer serves all calls on a stream).  Grown outside graph
    capture only: warm a captured call up once first.  A buffer that is
    replaced by a larger one stays allocated, so graphs captured on it remain
    valid (each keeps its own counters zero between replays)."""
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    ws = _WORKSPACE.get(idx)
    if ws is None or ws.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("the shared workspace must grow, which cannot happen during "
                               "graph capture: run the call once before capturing it")
        if ws is not None:
            _RETIRED.append(ws)
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _WORKSPACE[idx] = ws
    return ws


def _workspace_arg(size_fn, M, N, K, algo, dev, ws):
    """(pointer, bytes) of the workspace argument: None -> NULL (no split),
    "auto" -> the shared buffer, a tensor -> that tensor."""
    if ws is None:
        return ctypes.c_void_p(0), 0
    if isinstance(ws, str):
        if ws != "auto":
            raise ValueError(f"workspace must be None, 'auto' or a tensor (got {ws!r})")
        need = int(size_fn(M, N, K, ALGOS[algo]))
        if need == 0:
            return ctypes.c_void_p(0), 0
        ws = workspace(dev, need)
    if ws.device != dev or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the operands' device")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def _product(fn, name, a: TernaryPlanes, w: BinaryPlanes, out_dtype: str, algo: str,
             out: Optional[torch.Tensor], ws="auto", size_fn=None):
    if a.K != w.K:
        raise ValueError(f"K mismatch: activations {a.K}, weights {w.K}")
    if out_dtype not in _OUT_TORCH or algo not in ALGOS:
        raise ValueError(f"bad out_dtype {out_dtype!r} or algo {algo!r}")
    M = _check_ternary(a, "a")
    N = _check_binary(w, 1, "w")
    dev = a.mask.device
    if out is None:
        out = torch.empty((M, N), dtype=_OUT_TORCH[out_dtype], device=dev)
    _check_out(out, out_dtype, (M, N), dev)
    for t, n in ((a.sign, "a.sign"), (a.alpha, "a.alpha"), (a.nnz, "a.nnz"), (w.sign, "w.sign"),
                 (w.alpha, "w.alpha")):
        if t.device != dev:
            raise ValueError(f"{n} is on {t.device}, a.mask on {dev}")
    _dev_check(a.mask, "a.mask")
    wp, wb = _workspace_arg(size_fn, M, N, a.K, algo, dev, ws)
    _check(fn(_ptr(a.mask), _ptr(a.sign), _ptr(a.alpha), _ptr(a.nnz), _ptr(w.sign), _ptr(w.alpha),
              M, N, a.K, _ptr(out), DTYPES[out_dtype], out.stride(0), ALGOS[algo], wp, wb,
              _stream()), name)
    return out


def bwta_gemm(a: TernaryPlanes, w: BinaryPlanes, out_dtype: str = "f32", algo: str = "auto",
              out: Optional[torch.Tensor] = None, workspace="auto") -> torch.Tensor:
    """Y[M, N] = alpha_a * alpha_w * (t @ s^T) for the prefill linear.
    workspace: None (no cross-block split), "auto" (a shared zero-filled buffer)
    or a zero-initialised uint8 device tensor of bwta_gemm_workspace_size bytes."""
    L = lib()
    return _product(L.bwta_gemm, "bwta_gemm", a, w, out_dtype, algo, out, workspace,
                    L.bwta_gemm_workspace_size)


def bwta_gemv(a: TernaryPlanes, w: BinaryPlanes, out_dtype: str = "f32", algo: str = "auto",
              out: Optional[torch.Tensor] = None, workspace="auto") -> torch.Tensor:
    """Decode product for M <= 16 activation rows (workspace as for bwta_gemm)."""
    L = lib()
    return _product(L.bwta_gemv, "bwta_gemv", a, w, out_dtype, algo, out, workspace,
                    L.bwta_gemv_workspace_size)


def bwta_gemv_fused(X: torch.Tensor, w: BinaryPlanes, out_dtype: str = "f32",
                    out: Optional[torch.Tensor] = None, planes: bool = False,
                    workspace="auto"):
    """Decode linear in one launch: ternarize the rows of X [M, K] (fp32 or
    bf16, unit stride along K, M <= 16) and multiply them with w.  Returns Y, or
    (Y, TernaryPlanes) with planes=True (the kernel's ternarization of X).
    workspace="auto" takes the shared buffer at the size with which each row is
    ternarized once; None runs without one (every block ternarizes the rows)."""
    if X.dtype not in (torch.float32, torch.bfloat16) or X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D float32/bfloat16 tensor with unit stride along K")
    if out_dtype not in _OUT_TORCH:
        raise ValueError(f"bad out_dtype {out_dtype!r}")
    M, K = X.shape
    if w.K != K:
        raise ValueError(f"K mismatch: activations {K}, weights {w.K}")
    N = _check_binary(w, 1, "w")
    dev = X.device
    if out is None:
        out = torch.empty((M, N), dtype=_OUT_TORCH[out_dtype], device=dev)
    _check_out(out, out_dtype, (M, N), dev)
    if w.sign.device != dev:
        raise ValueError("X and w are on different devices")
    _dev_check(X, "X")
    tp = None
    if planes:
        rb = row_bytes(K)
        tp = TernaryPlanes(torch.empty((M, rb), dtype=torch.uint8, device=dev),
                           torch.empty((M, rb), dtype=torch.uint8, device=dev),
                           torch.empty(M, dtype=torch.float32, device=dev),
                           torch.empty(M, dtype=torch.int32, device=dev), K)
    L = lib()
    wp, wb = _workspace_arg(lambda m, n, k, _a: L.bwta_gemv_fused_workspace_size(m, n, k),
                            M, N, K, "mfma", dev, workspace)
    _check(L.bwta_gemv_fused(_ptr(X), _TORCH_DT[X.dtype], X.stride(0), _ptr(w.sign),
                             _ptr(w.alpha), M, N, K, _ptr(out), DTYPES[out_dtype], out.stride(0),
                             _ptr(tp.mask if tp else None), _ptr(tp.sign if tp else None),
                             _ptr(tp.alpha if tp else None), _ptr(tp.nnz if tp else None), wp, wb,
                             _stream()), "bwta_gemv_fused")
    return (out, tp) if planes else out


def bwta_gemv_fused_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().bwta_gemv_fused_workspace_size(M, N, K))


def set_fused_spin_limit(polls: int) -> None:
    """Test hook: polls of bwta_gemv_fused's bounded wait before a block
    ternarizes the rows itself (0: every block does; negative: the default)."""
    lib().bwta_set_fused_spin_limit(int(polls))


def bwta_gemv_noalloc(a: TernaryPlanes, w: BinaryPlanes, out_dtype: str = "f32",
                      algo: str = "auto", out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bwta_gemv on the library's own scratch array instead of a workspace (for
    callers that cannot allocate; pass `out` to allocate nothing here either)."""
    return _product(_noalloc_shim, "bwta_gemv_noalloc", a, w, out_dtype, algo, out, None, None)


def _noalloc_shim(*args):
    # _product passes (..., algo, workspace, ws_bytes, stream); the entry point
    # takes no workspace.
    return lib().bwta_gemv_noalloc(*args[:13], args[15])


def bwta_gemm_workspace_size(M: int, N: int, K: int, algo: str = "auto") -> int:
    return int(lib().bwta_gemm_workspace_size(M, N, K, ALGOS[algo]))


def bwta_gemv_workspace_size(M: int, N: int, K: int, algo: str = "auto") -> int:
    return int(lib().bwta_gemv_workspace_size(M, N, K, ALGOS[algo]))


def bwta_batched_gemm(batch: int, a: TernaryPlanes, a_batch_rows: int, b, b_batch_rows: int,
                      M: int, N: int, out_dtype: str = "f32", algo: str = "auto",
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Batched products for attention: B ternary (TernaryPlanes, e.g. Q K^T) or
    binary (BinaryPlanes, e.g. P V with V^T packed per channel).
    Returns Y [batch, M, N]."""
    K = a.K
    if b.K != K:
        raise ValueError("K mismatch")
    if out_dtype not in _OUT_TORCH or algo not in ALGOS:
        raise ValueError(f"bad out_dtype {out_dtype!r} or algo {algo!r}")
    a_rows = _check_ternary(a, "a")
    if isinstance(b, TernaryPlanes):
        b_rows = _check_ternary(b, "b")
        b_mask = b.mask
    else:
        b_rows = _check_binary(b, 1, "b")
        b_mask = None
    if batch > 0 and ((batch - 1) * a_batch_rows + M > a_rows or
                      (batch - 1) * b_batch_rows + N > b_rows):
        raise ValueError("the batch reaches past the rows of a or b")
    dev = a.mask.device
    if out is None:
        out = torch.empty((batch, M, N), dtype=_OUT_TORCH[out_dtype], device=dev)
    _check_out(out, out_dtype, (batch, M, N), dev)
    if tuple(out.shape) != (batch, M, N):
        raise ValueError("out must be [batch, M, N] with unit column stride")
    _dev_check(a.mask, "a.mask")
    if b.sign.device != dev:
        raise ValueError("a and b are on different devices")
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
    if out_dtype not in ("f32", "bf16"):
        raise ValueError(f"bad out_dtype {out_dtype!r}")
    rows = _check_ternary(q, "q")
    if heads <= 0 or rows % heads:
        raise ValueError("q rows must be heads * L")
    L = rows // heads
    if k.K != D or _check_ternary(k, "k") != rows:
        raise ValueError("k must match q: [heads * L, D]")
    if v.K != L or _check_binary(v, 1, "v") != heads * D:
        raise ValueError("v must be V^T planes [heads * D, L]")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    dev = q.mask.device
    if out is None:
        out = torch.empty((heads, L, D), dtype=_OUT_TORCH[out_dtype], device=dev)
    _check_out(out, out_dtype, (heads, L, D), dev)
    if tuple(out.shape) != (heads, L, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [heads, L, D] tensor")
    if k.mask.device != dev or v.sign.device != dev:
        raise ValueError("q, k and v are on different devices")
    _dev_check(q.mask, "q.mask")
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
    if out_dtype not in ("f32", "bf16"):
        raise ValueError(f"bad out_dtype {out_dtype!r} (two-plane products are scaled)")
    M = _check_ternary(a, "a")
    N2 = _check_binary(w, 1, "w")
    if N2 % 2:
        raise ValueError("two-plane weights have an even number of plane rows")
    N = N2 // 2
    dev = a.mask.device
    if out is None:
        out = torch.empty((M, N), dtype=_OUT_TORCH[out_dtype], device=dev)
    _check_out(out, out_dtype, (M, N), dev)
    if w.sign.device != dev:
        raise ValueError("a and w are on different devices")
    _dev_check(a.mask, "a.mask")
    _check(fn(_ptr(a.mask), _ptr(a.sign), _ptr(a.alpha), _ptr(a.nnz), _ptr(w.sign),
              _ptr(w.alpha), M, N, a.K, _ptr(out), DTYPES[out_dtype], out.stride(0), _stream()),
           name)
    return out
