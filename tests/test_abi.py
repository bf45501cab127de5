"""The C ABI of libbwta.so on the CPU: the library loads, exports every entry
point declared in include/bwta.h, and rejects bad arguments with the documented
status codes before anything reaches the GPU (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bwta.h")

OK, INVALID, ALIGN, UNSUPPORTED, HIPERR = range(5)
A = 0x10000          # a 16-byte aligned fake device address (never dereferenced)
MIS = 0x10004        # 4-byte aligned, not 16


@pytest.fixture(scope="module")
def L():
    from binary_ternary_matmul_amd import _binding, build
    if not os.path.exists(_binding.LIB_PATH):
        build.build()
    return _binding.lib()


def declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bwta_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"libbwta.so does not export {n}"


def test_probe_library_exports():
    """libbwta_probe.so (the benchmark's measurement kernels) exports what
    include/bwta_probe.h declares and rejects bad arguments before launching."""
    from binary_ternary_matmul_amd import build
    if not os.path.exists(build.PROBE_LIB):
        build.build()
    P = ctypes.CDLL(build.PROBE_LIB)
    names = declared_functions(os.path.join(ROOT, "include", "bwta_probe.h"))
    assert names == ["bwta_probe_mfma", "bwta_probe_stream_read"]
    for n in names:
        assert hasattr(P, n)
    V = ctypes.c_void_p
    P.bwta_probe_stream_read.argtypes = [V, ctypes.c_size_t, V, ctypes.c_int, V]
    P.bwta_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, V, V]
    assert P.bwta_probe_stream_read(V(A), 100, V(A), 0, V(0)) == -1    # not a multiple of 16
    assert P.bwta_probe_stream_read(V(A + 8), 64, V(A), 0, V(0)) == -1
    assert P.bwta_probe_mfma(2, 1024, 10, V(A), V(0)) == -1           # unknown format
    assert P.bwta_probe_mfma(0, 1022, 10, V(A), V(0)) == -1           # waves not in blocks of 4


def test_version_and_sizes(L):
    assert L.bwta_version() == 2
    for K, kp in [(1, 64), (64, 64), (65, 128), (768, 768), (11008, 11008), (100, 128)]:
        assert L.bwta_padded_k(K) == kp
        assert L.bwta_row_bytes(K) == kp // 8
    assert L.bwta_padded_k(0) == 0 and L.bwta_row_bytes(-5) == 0


def test_status_strings(L):
    for s, name in enumerate(["BWTA_OK", "BWTA_ERR_INVALID", "BWTA_ERR_ALIGN",
                              "BWTA_ERR_UNSUPPORTED", "BWTA_ERR_HIP"]):
        assert L.bwta_status_string(s).decode() == name


def gemm(L, fn="bwta_gemm", **kw):
    args = dict(a_mask=A, a_sign=A, a_alpha=A, a_nnz=A, w_sign=A, w_alpha=A, M=4, N=4, K=64,
                Y=A, y_dtype=0, ldy=4, algo=0, ws=0, ws_bytes=0)
    args.update(kw)
    f = getattr(L, fn)
    return f(*[ctypes.c_void_p(args[k]) if k in ("a_mask", "a_sign", "a_alpha", "a_nnz", "w_sign",
                                                  "w_alpha", "Y", "ws") else args[k]
               for k in ["a_mask", "a_sign", "a_alpha", "a_nnz", "w_sign", "w_alpha", "M", "N",
                         "K", "Y", "y_dtype", "ldy", "algo", "ws", "ws_bytes"]],
             ctypes.c_void_p(0))


@pytest.mark.parametrize("fn", ["bwta_gemm", "bwta_gemv"])
def test_product_validation(L, fn):
    assert gemm(L, fn, a_mask=0) == INVALID
    assert gemm(L, fn, w_sign=0) == INVALID
    assert gemm(L, fn, a_nnz=0) == INVALID
    assert gemm(L, fn, Y=0) == INVALID
    assert gemm(L, fn, K=0) == INVALID
    assert gemm(L, fn, K=-3) == INVALID
    assert gemm(L, fn, M=-1) == INVALID
    assert gemm(L, fn, ldy=3) == INVALID
    assert gemm(L, fn, y_dtype=7) == INVALID
    assert gemm(L, fn, algo=9) == INVALID
    assert gemm(L, fn, a_mask=MIS) == ALIGN
    assert gemm(L, fn, w_sign=A + 8) == ALIGN
    assert gemm(L, fn, a_alpha=A + 2) == ALIGN
    assert gemm(L, fn, Y=A + 1) == ALIGN
    assert gemm(L, fn, K=65537) == UNSUPPORTED
    assert b"K" in L.bwta_last_error()
    # empty products are a successful no-op, NULL pointers included
    assert gemm(L, fn, M=0) == OK
    assert gemm(L, fn, M=0, a_mask=0, Y=0) == OK
    assert gemm(L, fn, N=0, ldy=0) == OK
    # raw int32 output does not need the scales
    assert gemm(L, fn, a_alpha=0, w_alpha=0, y_dtype=2, M=0) == OK


def test_gemv_rejects_m_above_16(L):
    assert gemm(L, "bwta_gemv", M=17) == UNSUPPORTED
    assert b"16" in L.bwta_last_error()


def test_workspace_size_query(L):
    """The decode kernel splits K across blocks where it would otherwise split it
    inside a block: LLaMA2-70B down (N = 8192, K = 28672) from 8 rows on, not
    gate/up (1792 tiles of 16 rows) and not the M = 1 popcount kernel."""
    gv, gm = L.bwta_gemv_workspace_size, L.bwta_gemm_workspace_size
    AUTO, MFMA, POPC = 0, 1, 2
    need = gv(16, 8192, 28672, AUTO)
    assert need > 0 and need % 256 == 0
    assert need >= 512 * 16 * 16 * 4 * 2          # at least two int32 partial tiles each
    assert need <= (4 << 20) + (8 << 10)          # the stated cap on partials
    assert gv(8, 8192, 28672, AUTO) == need       # one tile of 16 rows holds M <= 16
    assert gv(4, 8192, 28672, AUTO) == 0          # below 8 rows the split does not pay
    assert gv(16, 8192, 28672, MFMA) == need
    assert gv(1, 8192, 28672, AUTO) == 0          # popcount GEMV
    assert gv(1, 8192, 28672, MFMA) == 0
    assert gv(16, 8192, 28672, POPC) == 0
    assert gv(16, 28672, 8192, AUTO) == 0         # enough tiles: no split
    assert gv(17, 8192, 28672, AUTO) == 0 and gv(0, 8192, 28672, AUTO) == 0
    assert gm(16, 8192, 28672, AUTO) == need      # bwta_gemm AUTO routes M <= 16 here
    assert gm(16, 8192, 28672, MFMA) == 0 and gm(64, 8192, 28672, AUTO) == 0


def test_fused_workspace_size_query(L):
    """The fused decode's workspace: the decode kernel's own bytes at least, the
    8 KiB counter region always (its last 256 bytes hold the row flags), plus the
    exchange planes (2 M row_bytes) and scales; 0 outside 1 <= M <= 16."""
    L.bwta_gemv_fused_workspace_size.restype = ctypes.c_size_t
    L.bwta_gemv_fused_workspace_size.argtypes = [ctypes.c_int64] * 3
    L.bwta_gemv_workspace_size.restype = ctypes.c_size_t
    L.bwta_gemv_workspace_size.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_int32]
    fz, gv = L.bwta_gemv_fused_workspace_size, L.bwta_gemv_workspace_size
    for M, N, K in [(16, 8192, 28672), (4, 28672, 8192), (1, 100, 1), (9, 600, 36928)]:
        rb = (K + 63) // 64 * 8
        need = fz(M, N, K)
        assert need % 256 == 0
        assert need >= max(gv(M, N, K, 1), 8192) + 2 * M * rb + 8 * M
        assert need <= max(gv(M, N, K, 1), 8192) + 2 * (M * rb + 255) + 512
    assert fz(0, 8192, 28672) == 0 and fz(17, 8192, 28672) == 0 and fz(4, 0, 8192) == 0
    assert fz(4, 8192, 0) == 0
    L.bwta_set_fused_spin_limit.restype = None
    L.bwta_set_fused_spin_limit.argtypes = [ctypes.c_int32]
    L.bwta_set_fused_spin_limit(0)
    L.bwta_set_fused_spin_limit(-1)  # back to the default


@pytest.mark.parametrize("fn", ["bwta_gemm", "bwta_gemv"])
def test_workspace_validation(L, fn):
    shape = dict(M=16, N=8192, K=28672, ldy=8192)
    need = getattr(L, fn + "_workspace_size")(16, 8192, 28672, 0)
    assert gemm(L, fn, ws=A, ws_bytes=need - 1, **shape) == INVALID
    assert b"workspace" in L.bwta_last_error()
    assert gemm(L, fn, ws=A + 16, ws_bytes=need, **shape) == ALIGN
    # a shape that does not use it ignores size and alignment
    assert gemm(L, fn, ws=A + 16, ws_bytes=0, M=0) == OK


def test_pack_validation(L):
    P = ctypes.c_void_p
    f = L.bwta_pack_weights
    assert f(P(0), 0, 4, 64, 64, 1, P(A), P(A), P(0)) == INVALID
    assert f(P(A), 5, 4, 64, 64, 1, P(A), P(A), P(0)) == INVALID
    assert f(P(A), 0, 4, 0, 64, 1, P(A), P(A), P(0)) == INVALID
    assert f(P(A), 0, 4, 64, 64, 0, P(A), P(A), P(0)) == INVALID
    assert f(P(A), 0, 4, 64, 64, 1, P(MIS), P(A), P(0)) == ALIGN
    assert f(P(A + 2), 0, 4, 64, 64, 1, P(A), P(A), P(0)) == ALIGN
    assert f(P(A + 2), 1, 0, 64, 64, 1, P(A), P(A), P(0)) == OK      # bf16: 2-byte aligned is fine
    assert f(P(A), 0, 0, 64, 64, 1, P(A), P(A), P(0)) == OK          # zero rows
    assert f(P(0), 0, 0, 64, 64, 1, P(0), P(0), P(0)) == OK          # zero rows, NULL pointers
    t = L.bwta_ternarize_pack
    assert t(P(A), 0, 4, 64, 64, P(A), P(A), P(A), P(0), P(0)) == INVALID   # nnz NULL
    assert t(P(A), 0, 4, 64, 32, P(A), P(A), P(A), P(A), P(0)) == INVALID   # stride < K
    assert t(P(A), 0, 4, 70000, 70000, P(A), P(A), P(A), P(A), P(0)) == UNSUPPORTED
    assert t(P(A), 0, 4, 64, 64, P(A), P(MIS), P(A), P(A), P(0)) == ALIGN
    assert t(P(A), 0, 0, 64, 64, P(A), P(A), P(A), P(A), P(0)) == OK


def test_batched_validation(L):
    P = ctypes.c_void_p
    f = L.bwta_batched_gemm

    def call(batch=2, b_mask=A, a_nnz=A, ab=4, bb=4, M=4, N=4, K=64, ldy=4, ys=16, dt=2):
        return f(batch, P(A), P(A), P(A), P(a_nnz), ab, P(b_mask), P(A), P(A), bb, M, N, K, P(A),
                 dt, ldy, ys, 0, P(0))
    assert call(batch=-1) == INVALID
    assert call(ab=-1) == INVALID
    assert call(b_mask=MIS) == ALIGN
    assert call(batch=70000) == UNSUPPORTED
    assert call(batch=0) == OK
    # empty batch: a no-op before any pointer is examined
    assert call(a_nnz=0, b_mask=0, batch=0) == OK
    # ternary x ternary does not use nnz; binary B does
    assert call(a_nnz=0, b_mask=0, M=0) == OK
    assert call(a_nnz=0, b_mask=0, K=0) == INVALID


def test_attention_validation(L):
    P = ctypes.c_void_p
    f = L.bwta_attention

    def call(heads=2, Lk=2048, D=128, q_mask=A, k_alpha=A, v_sign=A, O=A, dt=0, scale=0.088,
             p_out=0, p_mask=0, p_alpha=0, p_nnz=0):
        return f(heads, Lk, D, P(q_mask), P(A), P(A), P(A), P(A), P(k_alpha), P(v_sign), P(A),
                 ctypes.c_float(scale), P(O), dt, P(p_out), P(p_mask), P(p_alpha), P(p_nnz), P(0))
    assert call(heads=-1) == INVALID
    assert call(Lk=-2048) == INVALID
    assert call(dt=2) == INVALID                     # int32 output is not offered
    assert call(scale=float("inf")) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(heads=0) == OK                       # no-op before any pointer is examined
    assert call(heads=0, q_mask=0, O=0) == OK
    assert call(D=64) == UNSUPPORTED
    assert call(Lk=4096) == UNSUPPORTED
    assert call(Lk=1000) == UNSUPPORTED
    assert call(heads=70000) == UNSUPPORTED
    assert call(q_mask=0) == INVALID
    assert call(O=0) == INVALID
    assert call(v_sign=MIS) == ALIGN
    assert call(k_alpha=MIS) == ALIGN
    assert call(p_out=MIS) == ALIGN
    assert call(p_mask=MIS) == ALIGN
    assert call(p_nnz=A + 2) == ALIGN


def test_residual_validation(L):
    P = ctypes.c_void_p
    pk = L.bwta_pack_weights_residual
    assert pk(P(A), 0, 33, 64, 64, P(A), P(A), P(0)) == UNSUPPORTED   # rows not a multiple of 32
    assert pk(P(A), 5, 32, 64, 64, P(A), P(A), P(0)) == INVALID       # dtype
    assert pk(P(A), 0, 32, 0, 64, P(A), P(A), P(0)) == INVALID        # K
    assert pk(P(A), 0, 32, 64, 32, P(A), P(A), P(0)) == INVALID       # stride < K
    assert pk(P(A), 0, 32, 64, 64, P(MIS), P(A), P(0)) == ALIGN
    assert pk(P(0), 0, 0, 64, 64, P(0), P(0), P(0)) == OK            # no rows
    g = L.bwta_gemm_residual

    def call(M=4, N=64, K=128, Y=A, dt=0, ldy=64, w_sign=A, a_nnz=0):
        return g(P(A), P(A), P(A), P(a_nnz), P(w_sign), P(A), M, N, K, P(Y), dt, ldy, P(0))
    assert call(N=48) == UNSUPPORTED
    assert call(M=-1) == INVALID
    assert call(K=0) == INVALID
    assert call(dt=2) == INVALID                                      # scaled outputs only
    assert call(ldy=32) == INVALID
    assert call(w_sign=MIS) == ALIGN
    assert call(Y=0) == INVALID
    assert call(M=0) == OK
    assert call(M=0, Y=0, w_sign=0) == OK
    v = L.bwta_gemv_residual

    def callv(M=4, N=64, K=128, Y=A, dt=0, ldy=64, a_nnz=A):
        return v(P(A), P(A), P(A), P(a_nnz), P(A), P(A), M, N, K, P(Y), dt, ldy, P(0))
    assert callv(M=17) == UNSUPPORTED
    assert callv(N=40) == UNSUPPORTED
    assert callv(a_nnz=0) == INVALID                                   # the decode path needs nnz
    assert callv(dt=2) == INVALID
    assert callv(M=0, Y=0) == OK


def test_binding_refuses_host_tensors():
    import torch
    from binary_ternary_matmul_amd import bwta_ternarize_pack
    with pytest.raises(ValueError):
        bwta_ternarize_pack(torch.zeros(4, 64))
