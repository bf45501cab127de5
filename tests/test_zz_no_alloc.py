"""bwta_gemv_noalloc (the decode product on the library's own scratch array)
against bwta_gemv with a caller-owned workspace, through the C ABI.

Calls in a row on one stream: the LLaMA2-70B down shape at M = 16 (a 4-way
cross-block K split over 512 tiles), then a smaller input (fewer rows, tiles
and K), then the first shape again, so the scratch array's counters must come
back to zero after each call.  Bar: int32 accumulators, fp32 and bf16 outputs
bit-identical to bwta_gemv's, which the oracle also checks here."""
import ctypes

import numpy as np
import pytest

from binary_ternary_matmul_amd import inputs
from tests.helpers import to_dev, to_host

pytestmark = pytest.mark.gpu

DT = {"f32": 0, "bf16": 1, "i32": 2}


@pytest.fixture(scope="module")
def bw():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import binary_ternary_matmul_amd as b
    b.lib()
    return b


def _case(M, N, K, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = inputs.f32_to_bf16_bits(inputs.student_t(rng, (M, K), 3.0))
    w = inputs.normal(rng, (N, K), 0.015)
    return x, w


def _noalloc(bw, a, wp, out, out_dtype):
    """Call the entry point directly through ctypes (no workspace argument)."""
    import torch
    L = bw.lib()
    M, N = a.mask.shape[0], wp.sign.shape[0]
    P = ctypes.c_void_p
    st = L.bwta_gemv_noalloc(P(a.mask.data_ptr()), P(a.sign.data_ptr()), P(a.alpha.data_ptr()),
                             P(a.nnz.data_ptr()), P(wp.sign.data_ptr()), P(wp.alpha.data_ptr()),
                             M, N, a.K, P(out.data_ptr()), DT[out_dtype], out.stride(0), 0,
                             P(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.bwta_last_error().decode()
    return out


def test_gemv_noalloc_matches_gemv(bw, oracle):
    import torch
    cases = [(16, 8192, 28672, 11), (8, 3000, 17000, 12), (16, 8192, 28672, 13)]
    for i, (M, N, K, seed) in enumerate(cases):
        need = bw.bwta_gemv_workspace_size(M, N, K)
        assert need > 0, "the case must run the split that uses the scratch array"
        x, w = _case(M, N, K, seed)
        a = bw.bwta_ternarize_pack(to_dev(x))
        wp = bw.bwta_pack_weights(to_dev(w))
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        for out_dtype, tdt in (("i32", torch.int32), ("f32", torch.float32),
                               ("bf16", torch.bfloat16)):
            ref = to_host(bw.bwta_gemv(a, wp, out_dtype, "auto", workspace=ws))
            out = torch.full((M, N), 7, dtype=tdt, device="cuda")
            got = to_host(_noalloc(bw, a, wp, out, out_dtype))
            bits = np.uint16 if out_dtype == "bf16" else np.uint32
            assert (got.view(bits) == ref.view(bits)).all(), \
                f"call {i} ({M}x{N}x{K}, {out_dtype}): outputs differ from bwta_gemv"
            if out_dtype == "i32":
                t, _, _ = oracle.ternarize(x)
                s, _ = oracle.binarize(w)
                assert (got == oracle.matmul_i32(t, s, threads=16)).all(), f"call {i}: vs oracle"
