"""Benchmark of the binary-weight x ternary-activation hot path on one MI355X.

One step = one LLaMA-7B-shaped decoder layer's linears at prefill (M = 2048
tokens): ternarize+pack the four bf16 activation inputs (attention input,
attention output, MLP input, MLP activation) and run the seven binary x ternary
linears (q, k, v, o: 4096 -> 4096; gate, up: 4096 -> 11008; down: 11008 -> 4096)
with the fused bf16 epilogue, as four products: the projections that read the same
input have their packed weights stacked along N (qkv 4096 -> 12288, gate_up
4096 -> 22016), which gives the same outputs as separate products.  Weights are
packed once before timing (as for a deployed model).  `value` is the step's
int8-equivalent throughput in TOPS (2*M*N*K over the seven linears per step time,
ternarize included).

The same run also measures, each in its own object on the JSON line:
  gemv       decode GEMV/skinny GEMM, LLaMA2-70B shapes, M in {1, 4, 16}: HBM GB/s
             with >= 20 rotating weight copies so every launch reads from HBM
  attention  32 heads x 2048 x 128: ternarize Q, K -> Q K^T (int32 scores) and
             ternarize P -> pack V^T -> P V
  mfma_i8    the int8 MFMA GEMM on the same products (the FP4 kernel's alternative)
  popcount   the VALU popcount GEMM on the same products (the alternative to MFMA)
  bert       BERT-base encoder linears, M = 4096, fp32 in, bf16 out
  roofline   the FP4 MFMA GEMM kernel's achieved TOPS against the dense FP4 peak
             (gemm_frac_of_int8_peak gives the same against the int8 peak)
  cpu_baseline  the scalar CPU oracle on a bounded row sample of the same step

Inputs are synthetic (seeded generators in binary_ternary_matmul_amd.inputs).
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POPS
FP4_PEAK_TOPS = 10100.0      # MI355X dense FP4 MFMA, 10.1 PFLOP/s (the GEMM kernel's dtype)
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz: 32-bit VALU lane-operations per second
# (one wave64 instruction takes 4 cycles on a 16-lane SIMD; packed fp32 not counted).
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9
VALU_OPS_PER_SCORE = 11


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(x):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def graph_of(fn, reps=1, warm=2):
    """Capture `reps` back-to-back calls of fn (all launches on torch's current
    stream) into one HIP graph.  Many calls per graph amortise the graph-launch
    overhead, which on this stack is several microseconds per replay."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(warm):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, reps_inside, replays=3):
    """Milliseconds per captured call: HIP events around `replays` replays of a
    graph holding `reps_inside` calls."""
    import torch
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(replays):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / (replays * reps_inside)


def time_calls(fn, reps=20, replays=3):
    return time_graph(graph_of(fn, reps), reps, replays)


def profiled_traffic(key):
    """HBM bytes per launch of kernel `key` from the rocprofv3 FETCH_SIZE /
    WRITE_SIZE summaries under profiles/ (a line 'traffic <key> bytes_per_launch=..
    source=<file> sha256=<hex>'), or None when no summary names the key or its
    kernel source has changed since the counters were taken."""
    import glob
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    for path in sorted(glob.glob(os.path.join(root, "profiles", "*.md"))):
        with open(path) as f:
            for ln in f:
                parts = ln.split()
                if len(parts) < 3 or parts[0] != "traffic" or parts[1] != key:
                    continue
                kv = dict(p.split("=", 1) for p in parts[2:] if "=" in p)
                try:
                    with open(os.path.join(root, kv["source"]), "rb") as src:
                        if hashlib.sha256(src.read()).hexdigest() != kv["sha256"]:
                            return None
                    return {"bytes": int(kv["bytes_per_launch"]),
                            "algorithmic_bytes": int(kv["algorithmic_bytes_per_launch"]),
                            "summary": os.path.relpath(path, root)}
                except (KeyError, OSError, ValueError):
                    return None
    return None


def probe_read_us(x, reps=20):
    """Time of the read-only stream probe over the bytes of device tensor x, read
    again and again (as a benchmark loop re-reads the same input)."""
    import ctypes
    import torch
    from binary_ternary_matmul_amd import build
    P = ctypes.CDLL(build.PROBE_LIB)
    V = ctypes.c_void_p
    P.bwta_probe_stream_read.argtypes = [V, ctypes.c_size_t, V, ctypes.c_int, V]
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    nb = x.numel() * x.element_size() // 16 * 16
    # the stream is read inside the call: time_calls captures on its own stream
    best = None
    for blocks in (0, 1024, 2048, 4096):
        ms = time_calls(lambda blocks=blocks: P.bwta_probe_stream_read(
            V(x.data_ptr()), nb, V(sink.data_ptr()), blocks,
            V(torch.cuda.current_stream().cuda_stream)), reps=reps)
        best = ms if best is None else min(best, ms)
    return best * 1e3


def ceilings(copies=24):
    """The chip's measured ceilings (libbwta_probe.so): read-only HBM streams of
    one decode weight's size (29.59 MB, each launch reading another of `copies`
    buffers so that it comes from HBM) and of 1 GiB, and matrix-core loops of
    16 independent FP4 (e2m1) and int8 products per wave on all 1024 SIMDs."""
    import ctypes
    import torch
    from binary_ternary_matmul_amd import build
    P = ctypes.CDLL(build.PROBE_LIB)
    V = ctypes.c_void_p
    P.bwta_probe_stream_read.argtypes = [V, ctypes.c_size_t, V, ctypes.c_int, V]
    P.bwta_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, V, V]
    st = lambda: V(torch.cuda.current_stream().cuda_stream)
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    out = {}
    nb = 29591552                                      # 70B gate/up decode bytes, rounded to 16
    bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    for b in bufs:
        b.fill_(1)

    # The grid is swept (0 = one round of loads per thread) and the fastest kept.
    grids = (0, 1024, 2048, 4096)

    def small(blocks):
        for b in bufs:
            assert P.bwta_probe_stream_read(V(b.data_ptr()), nb, V(sink.data_ptr()), blocks,
                                            st()) == 0
    ms = min(time_calls(lambda g=g: small(g), reps=2) for g in grids) / copies
    out["hbm_read_29.6MB_GBps"] = round(nb / (ms * 1e-3) / 1e9, 1)
    del bufs
    big = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    ms = min(time_calls(lambda g=g: P.bwta_probe_stream_read(V(big.data_ptr()), big.numel(),
                                                              V(sink.data_ptr()), g, st()), reps=3)
             for g in (0, 2048, 4096, 8192))
    out["hbm_read_1GiB_GBps"] = round(big.numel() / (ms * 1e-3) / 1e9, 1)
    del big
    for fmt, name, per in ((0, "fp4_mfma_loop_TOPS", 131072), (1, "int8_mfma_loop_TOPS", 65536)):
        iters = 1500
        ms = time_calls(lambda fmt=fmt: P.bwta_probe_mfma(fmt, 1024, iters, V(sink.data_ptr()),
                                                          st()), reps=3)
        out[name] = round(1024 * iters * 16 * per / (ms * 1e-3) / 1e12, 1)
    return out


def bench_prefill(bw, steps, warmup, M=2048):
    import torch
    from binary_ternary_matmul_amd import inputs
    acts, lins = inputs.llama7b_products(M)
    log(f"[prefill] generating inputs M={M}")
    X = {name: dev(gen()) for name, gen in acts.items()}
    W = {}
    for lin in lins:
        W[lin.name] = bw.bwta_pack_weights(dev(lin.w()))
    torch.cuda.synchronize()
    outs = {lin.name: torch.empty((M, lin.N), dtype=torch.bfloat16, device="cuda") for lin in lins}
    ops = sum(2.0 * M * lin.N * lin.K for lin in lins)

    def ternarize_all():
        return {name: bw.bwta_ternarize_pack(x) for name, x in X.items()}

    def gemms(planes):
        for lin in lins:
            a = planes[inputs.LLAMA7B_INPUTS[lin.name]]
            bw.bwta_gemm(a, W[lin.name], "bf16", "mfma", outs[lin.name])

    def step():
        # in layer order: each input is ternarized right before the product that
        # reads it (as a decoder layer produces them), so its planes are warm
        for lin in lins:
            a = bw.bwta_ternarize_pack(X[inputs.LLAMA7B_INPUTS[lin.name]])
            bw.bwta_gemm(a, W[lin.name], "bf16", "mfma", outs[lin.name])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # The timed region is one HIP graph holding exactly `steps` steps: the same
    # kernels the eager calls launch, without per-launch host overhead.
    g_steps = graph_of(step, reps=steps)
    torch.cuda.synchronize()
    s_ev = torch.cuda.Event(enable_timing=True)
    e_ev = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s_ev.record()
    g_steps.replay()
    e_ev.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = s_ev.elapsed_time(e_ev) / steps
    # GEMM-only time (the dominant kernel) and a per-GEMM breakdown.
    planes = ternarize_all()
    gemm_ms = time_calls(lambda: gemms(planes), reps=steps)
    per_gemm = {}
    for lin in lins:
        a = planes[inputs.LLAMA7B_INPUTS[lin.name]]
        ms = time_calls(lambda a=a, lin=lin: bw.bwta_gemm(a, W[lin.name], "bf16", "mfma",
                                                          outs[lin.name]), reps=steps)
        per_gemm[lin.name] = {"M": M, "N": lin.N, "K": lin.K, "us": round(ms * 1e3, 2),
                              "tops": round(2.0 * M * lin.N * lin.K / (ms * 1e-3) / 1e12, 1)}
    tern_ms = time_calls(ternarize_all, reps=steps)
    # Ternarize roofline (HBM-bound): each input's bf16 rows read once, both
    # planes and the per-row alpha and nnz written once.
    tern = {}
    tern_bytes = 0
    for name, x in X.items():
        rows, K = x.shape
        nb = rows * K * x.element_size() + rows * (2 * bw.row_bytes(K) + 8)
        tern_bytes += nb
        ms = time_calls(lambda x=x: bw.bwta_ternarize_pack(x), reps=steps)
        tern[name] = {"rows": rows, "K": K, "us": round(ms * 1e3, 2), "bytes": nb,
                      "GBps": round(nb / (ms * 1e-3) / 1e9, 1)}
    tern_gbs = tern_bytes / (tern_ms * 1e-3) / 1e9
    tern_roof = {"bound": "hbm", "kernel": "pack_rows_kernel", "achieved": round(tern_gbs, 1),
                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(tern_gbs / HBM_PEAK_GBS, 3),
                 "bytes_per_step": tern_bytes, "traffic": None, "per_input": tern}
    trs = [profiled_traffic(f"pack_rows_kernel.ternarize.K{t['K']}") for t in tern.values()]
    if all(trs):
        tern_roof["traffic"] = sum(t["bytes"] for t in trs)
        tern_roof["traffic_source"] = trs[0]["summary"]
    return dict(ops=ops, ms_step=ms_step, wall_ms_step=wall * 1e3 / steps, gemm_ms=gemm_ms,
                ternarize_ms=tern_ms, ternarize_roofline=tern_roof, per_gemm=per_gemm, lins=lins,
                X=X, W=W, M=M)


def bench_algo(bw, pre, algo, reps=5):
    """The same four products with another kernel family (popcount, int8 MFMA)."""
    import torch
    from binary_ternary_matmul_amd import inputs
    planes = {name: bw.bwta_ternarize_pack(x) for name, x in pre["X"].items()}
    res = {}
    tot_ops, tot_ms = 0.0, 0.0
    for lin in pre["lins"]:
        a = planes[inputs.LLAMA7B_INPUTS[lin.name]]
        out = torch.empty((pre["M"], lin.N), dtype=torch.bfloat16, device="cuda")
        ms = time_calls(lambda a=a, lin=lin: bw.bwta_gemm(a, pre["W"][lin.name], "bf16", algo,
                                                          out), reps=reps)
        ops = 2.0 * pre["M"] * lin.N * lin.K
        tot_ops += ops
        tot_ms += ms
        res[lin.name] = {"us": round(ms * 1e3, 1), "tops": round(ops / (ms * 1e-3) / 1e12, 1)}
    return {"layer_tops": round(tot_ops / (tot_ms * 1e-3) / 1e12, 1),
            "layer_frac_of_int8_peak": round(tot_ops / (tot_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 3),
            "fp4_mfma_speedup": round(tot_ms / pre["gemm_ms"], 2), "per_gemm": res}


def bench_residual(bw, pre, reps=5):
    """The same four products with two-plane residual weights (bwta_gemm_residual):
    both planes in one pass; ops counted per plane (twice the single-plane ops)."""
    import torch
    from binary_ternary_matmul_amd import inputs
    acts, lins = inputs.llama7b_products(pre["M"])
    planes = {name: bw.bwta_ternarize_pack(x) for name, x in pre["X"].items()}
    res, tot_ops, tot_ms = {}, 0.0, 0.0
    for lin in lins:
        wr = bw.bwta_pack_weights_residual(dev(lin.w()))
        a = planes[inputs.LLAMA7B_INPUTS[lin.name]]
        out = torch.empty((pre["M"], lin.N), dtype=torch.bfloat16, device="cuda")
        ms = time_calls(lambda a=a, wr=wr, out=out: bw.bwta_gemm_residual(a, wr, "bf16", out),
                        reps=reps)
        ops = 2 * 2.0 * pre["M"] * lin.N * lin.K
        tot_ops += ops
        tot_ms += ms
        res[lin.name] = {"us": round(ms * 1e3, 1), "tops": round(ops / (ms * 1e-3) / 1e12, 1),
                         "vs_one_plane": round(ms / (pre["per_gemm"][lin.name]["us"] * 1e-3), 2)}
        del wr
    return {"layer_ms": round(tot_ms, 4), "layer_tops_two_planes": round(tot_ops / (tot_ms * 1e-3) / 1e12, 1),
            "time_vs_one_plane": round(tot_ms / pre["gemm_ms"], 2), "per_gemm": res}


def bench_gemv_residual(bw, copies=12, reps=3):
    """Decode with two-plane residual weights (bwta_gemv_residual): HBM GB/s over
    rotating copies of both planes (> 350 MB per shape)."""
    import torch
    from binary_ternary_matmul_amd import inputs
    out = {}
    for shape in ("gate_up", "down"):
        lin16 = [l for l in inputs.llama70b_decode(16) if l.name == shape][0]
        wr = bw.bwta_pack_weights_residual(dev(lin16.w()))
        ws = [wr] + [bw.ResidualPlanes(wr.sign.clone(), wr.alpha.clone(), wr.K)
                     for _ in range(copies - 1)]
        for M in (1, 4, 16):
            lin = [l for l in inputs.llama70b_decode(M) if l.name == shape][0]
            a = bw.bwta_ternarize_pack(dev(lin.x()))
            y = torch.empty((M, lin.N), dtype=torch.float32, device="cuda")

            def run(a=a, y=y):
                for w in ws:
                    bw.bwta_gemv_residual(a, w, "f32", y)
            us = time_calls(run, reps=reps) * 1e3 / len(ws)
            kp = bw.padded_k(lin.K)
            nbytes = 2 * lin.N * kp / 8 + 8 * lin.N + M * (2 * kp / 8 + 8) + 4 * M * lin.N
            gbs = nbytes / (us * 1e-6) / 1e9
            kern = "gemv_popcount_kernel" if M == 1 else "gemv_mfma_kernel"  # two-plane modes
            out[f"{shape}_M{M}"] = {"N": lin.N, "K": lin.K, "kernel": kern,
                                    "us": round(us, 2), "bytes": int(nbytes), "GBps": round(gbs, 1),
                                    "hbm_frac": round(gbs / HBM_PEAK_GBS, 3)}
        del ws, wr
    return out


def bench_gemv(bw, copies=24, reps=4):
    """Decode: HBM GB/s with rotating packed-weight copies (> 512 MB per shape)."""
    import torch
    from binary_ternary_matmul_amd import inputs
    out = {}
    for M in (1, 4, 16):
        for lin in inputs.llama70b_decode(M):
            if M == 1:
                log(f"[gemv] packing {lin.name} {lin.N}x{lin.K}")
                w = bw.bwta_pack_weights(dev(lin.w()))
                torch.cuda.synchronize()
                ws = [w] + [bw.BinaryPlanes(w.sign.clone(), w.alpha.clone(), w.K)
                            for _ in range(copies - 1)]
                out.setdefault("_w", {})[lin.name] = ws
            ws = out["_w"][lin.name]
            a = bw.bwta_ternarize_pack(dev(lin.x()))
            y = torch.empty((M, lin.N), dtype=torch.float32, device="cuda")

            def run_all(a=a, y=y, ws=ws):
                for wi in ws:
                    bw.bwta_gemv(a, wi, "f32", "auto", y)
            ms = time_calls(run_all, reps=reps)
            us = ms * 1e3 / len(ws)
            kp = bw.padded_k(lin.K)
            nbytes = lin.N * kp / 8 + 4 * lin.N + M * (2 * kp / 8 + 8) + 4 * M * lin.N
            gbs = nbytes / (us * 1e-6) / 1e9
            kern = "gemv_popcount_kernel" if M == 1 else "gemv_mfma_kernel"  # algo "auto"
            tr = profiled_traffic(f"{kern}.{lin.name}.M{M}")
            out[f"{lin.name}_M{M}"] = {"N": lin.N, "K": lin.K, "kernel": kern, "us": round(us, 2),
                                       "bytes": int(nbytes), "GBps": round(gbs, 1),
                                       "hbm_frac": round(gbs / HBM_PEAK_GBS, 3),
                                       "traffic": tr["bytes"] if tr else None}
        # Gate and up of one MLP stacked into one [57344, 8192] weight: one launch
        # reads both (the same bytes as two launches, half the fixed costs).
        if M == 1:
            log("[gemv] packing up 28672x8192 (gate/up stacked)")
            up = bw.bwta_pack_weights(dev(inputs.llama70b_up_weight()()))
            out["_w"]["gate_up_fused"] = [
                bw.BinaryPlanes(torch.cat([g.sign, up.sign]), torch.cat([g.alpha, up.alpha]), g.K)
                for g in out["_w"]["gate_up"]]
            del up
        ws = out["_w"]["gate_up_fused"]
        lin = [l for l in inputs.llama70b_decode(M) if l.name == "gate_up"][0]
        a = bw.bwta_ternarize_pack(dev(lin.x()))
        N2 = 2 * lin.N
        y = torch.empty((M, N2), dtype=torch.float32, device="cuda")

        def run_fused(a=a, y=y, ws=ws):
            for wi in ws:
                bw.bwta_gemv(a, wi, "f32", "auto", y)
        ms = time_calls(run_fused, reps=reps)
        us = ms * 1e3 / len(ws)
        kp = bw.padded_k(lin.K)
        nbytes = N2 * kp / 8 + 4 * N2 + M * (2 * kp / 8 + 8) + 4 * M * N2
        gbs = nbytes / (us * 1e-6) / 1e9
        kern = "gemv_popcount_kernel" if M == 1 else "gemv_mfma_kernel"
        tr = profiled_traffic(f"{kern}.gate_up_fused.M{M}")
        out[f"gate_up_fused_M{M}"] = {"N": N2, "K": lin.K, "kernel": kern, "us": round(us, 2),
                                      "bytes": int(nbytes), "GBps": round(gbs, 1),
                                      "hbm_frac": round(gbs / HBM_PEAK_GBS, 3),
                                      "traffic": tr["bytes"] if tr else None}
    # The decode linear end to end (one step of a decoder: bf16 activations in),
    # per shape and M: ternarize + bwta_gemv as two launches, and bwta_gemv_fused
    # (one launch that ternarizes inside the decode kernel).
    e2e = {}
    for M in (1, 4, 16):
        for lin in inputs.llama70b_decode(M):
            ws = out["_w"][lin.name]
            X = dev(lin.x())
            y = torch.empty((M, lin.N), dtype=torch.float32, device="cuda")

            def two(X=X, y=y, ws=ws):
                for wi in ws:
                    bw.bwta_gemv(bw.bwta_ternarize_pack(X), wi, "f32", "auto", y)

            def fused(X=X, y=y, ws=ws):
                for wi in ws:
                    bw.bwta_gemv_fused(X, wi, "f32", y)
            u2 = time_calls(two, reps=reps) * 1e3 / len(ws)
            uf = time_calls(fused, reps=reps) * 1e3 / len(ws)
            e2e[f"{lin.name}_M{M}"] = {"ternarize_plus_gemv_us": round(u2, 2),
                                       "fused_us": round(uf, 2),
                                       "faster": "fused" if uf < u2 else "two_launches"}
    out["decode_linear_end_to_end"] = e2e
    out.pop("_w", None)
    # The decode kernel's roofline on the gate/up shape at M = 1 (the popcount
    # GEMV that AUTO runs there): algorithmic bytes per launch over the measured
    # per-launch time.
    ref = out.get("gate_up_M1")
    if ref:
        tr = profiled_traffic("gemv_popcount_kernel.gate_up.M1")
        out["roofline"] = {"bound": "hbm", "kernel": ref["kernel"], "shape": "gate_up_M1",
                           "achieved": ref["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": ref["hbm_frac"], "traffic": tr["bytes"] if tr else None}
    return out


def bench_attention(bw, reps=5, H=32, L=2048, D=128):
    import torch
    from binary_ternary_matmul_amd import inputs
    att = inputs.attention(H, L, D)
    Q = dev(att.q.reshape(H * L, D))
    Kt = dev(att.k.reshape(H * L, D))
    # V as [L, H*D] (tokens x all heads' channels): one launch packs V^T of every
    # head, plane row h*D + d = channel d of head h.
    Vf = dev(np.ascontiguousarray(att.v.transpose(1, 0, 2).reshape(L, H * D)))
    scores = torch.empty((H, L, L), dtype=torch.int32, device="cuda")
    O = torch.empty((H, L, D), dtype=torch.float32, device="cuda")
    # P for timing: softmax of the scaled scores, computed once on the GPU with torch
    qa = bw.bwta_ternarize_pack(Q)
    ka = bw.bwta_ternarize_pack(Kt)
    bw.bwta_batched_gemm(H, qa, L, ka, L, L, L, "i32", "auto", scores)
    z = scores.float() * (qa.alpha.view(H, L, 1) * ka.alpha.view(H, 1, L)) / (D ** 0.5)
    P = torch.softmax(z, dim=-1).reshape(H * L, L).contiguous()
    del z
    torch.cuda.synchronize()

    def qk():
        a = bw.bwta_ternarize_pack(Q)
        b = bw.bwta_ternarize_pack(Kt)
        bw.bwta_batched_gemm(H, a, L, b, L, L, L, "i32", "auto", scores)

    def pv():
        pa = bw.bwta_ternarize_pack(P)
        vb = bw.bwta_pack_weights(Vf, transpose=True)
        bw.bwta_batched_gemm(H, pa, L, vb, D, L, D, "f32", "auto", O)

    # Fused: Q K^T -> softmax -> ternarize P -> P V in one launch (no scores or P
    # in memory), timed alone on resident planes and with the packing of Q, K, V^T.
    vb = bw.bwta_pack_weights(Vf, transpose=True)
    Of = torch.empty((H, L, D), dtype=torch.float32, device="cuda")

    def fused():
        bw.bwta_attention(qa, ka, vb, H, out=Of)

    def fused_all():
        bw.bwta_attention(bw.bwta_ternarize_pack(Q), bw.bwta_ternarize_pack(Kt),
                          bw.bwta_pack_weights(Vf, transpose=True), H, out=Of)

    ms_qk = time_calls(qk, reps=reps)
    ms_pv = time_calls(pv, reps=reps)
    ms_f = time_calls(fused, reps=reps)
    ms_fa = time_calls(fused_all, reps=reps)
    ops = 2.0 * H * L * L * D
    rb = bw.row_bytes(D)
    qk_bytes = 2 * (H * L * D * 2) + 2 * 2 * (2 * H * L * rb + 8 * H * L) + H * L * L * 4
    return {"heads": H, "L": L, "d": D,
            "qk_ms": round(ms_qk, 3), "qk_scores_GBps": round(H * L * L * 4 / (ms_qk * 1e-3) / 1e9, 1),
            # Q K^T with ternarizing Q and K: bound by HBM, its algorithmic bytes are
            # the bf16 Q and K read, their planes and scales written and read back,
            # and the int32 scores written.
            "qk_roofline": {"bound": "hbm", "kernel": "gemm_mfma_kernel (+ pack_rows_kernel)",
                            "achieved": round(qk_bytes / (ms_qk * 1e-3) / 1e9, 1),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(qk_bytes / (ms_qk * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
                            "bytes": qk_bytes},
            "pv_ms": round(ms_pv, 3), "pv_tops_incl_ternarize_P": round(ops / (ms_pv * 1e-3) / 1e12, 1),
            "fused_kernel": "attention_kernel", "fused_ms": round(ms_f, 4),
            "fused_tops": round(2 * ops / (ms_f * 1e-3) / 1e12, 1),
            "fused_scores_per_s": round(H * L * L / (ms_f * 1e-3), -6),
            "fused_incl_packing_ms": round(ms_fa, 4),
            "unfused_over_fused": round((ms_qk + ms_pv) / ms_f, 2),
            # The fused kernel is bound by vector-ALU issue: the method's ~11 VALU
            # operations per score (scale, max, exp argument, exp, sum, normalise,
            # two tree adds, compare, select) against the chip's lane-operation rate.
            "fused_roofline": {"bound": "alu", "kernel": "attention_kernel",
                               "achieved": round(H * L * L * VALU_OPS_PER_SCORE / (ms_f * 1e-3)),
                               "peak": VALU_PEAK_LANE_OPS, "unit": "lane-op/s",
                               "frac": round(H * L * L * VALU_OPS_PER_SCORE / (ms_f * 1e-3)
                                             / VALU_PEAK_LANE_OPS, 3)}}


def bench_bert(bw, reps=10):
    """BERT-base encoder linears (M = 4096, fp32 in, bf16 out), each timed as
    ternarize + product.  Roofline: these sit near the ridge, so the bound is the
    larger of the HBM time of the algorithmic bytes (fp32 X read; activation
    planes and scales written and read back; weight plane and scales read; bf16
    Y written) and the FP4 matrix-core time of 2 M N K."""
    import torch
    from binary_ternary_matmul_amd import inputs
    lins = inputs.bert_encoder()
    tot_ops, tot_ms, tot_ideal = 0.0, 0.0, 0.0
    res = {}
    for lin in lins:
        x = dev(lin.x())
        w = bw.bwta_pack_weights(dev(lin.w()))
        y = torch.empty((lin.M, lin.N), dtype=torch.bfloat16, device="cuda")
        ms = time_calls(lambda x=x, w=w, y=y: bw.bwta_gemm(bw.bwta_ternarize_pack(x), w, "bf16",
                                                           "auto", y), reps=reps)
        ops = 2.0 * lin.M * lin.N * lin.K
        rb = bw.row_bytes(lin.K)
        nbytes = (lin.M * lin.K * 4 + 2 * (2 * lin.M * rb + 8 * lin.M) + lin.N * rb + 4 * lin.N
                  + lin.M * lin.N * 2)
        ideal_us = max(nbytes / (HBM_PEAK_GBS * 1e9), ops / (FP4_PEAK_TOPS * 1e12)) * 1e6
        tot_ops += ops
        tot_ms += ms
        tot_ideal += ideal_us
        res[lin.name] = {"us": round(ms * 1e3, 1), "tops": round(ops / (ms * 1e-3) / 1e12, 1),
                         "bytes": int(nbytes), "roofline_us": round(ideal_us, 2),
                         "frac": round(ideal_us / (ms * 1e3), 3)}
    return {"layer_tops_incl_ternarize": round(tot_ops / (tot_ms * 1e-3) / 1e12, 1),
            "roofline": {"bound": "max(hbm, mfma)", "achieved_us": round(tot_ms * 1e3, 1),
                         "roofline_us": round(tot_ideal, 1),
                         "frac": round(tot_ideal / (tot_ms * 1e3), 3)},
            "per_gemm": res}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(M=2048, rows=2048, rows_1t=32):
    """The oracle, untouched, on the same step: ternarize the four inputs and run
    the seven products as a dense int32 loop, on all host threads (at most 16,
    the cores a GPU machine gives one GPU) over all `rows` token rows, and on one
    thread over the first `rows_1t` rows (extrapolated to `rows`).  Each step is
    timed on its own."""
    from binary_ternary_matmul_amd import inputs
    from oracle import oracle
    acts, lins = inputs.llama7b_prefill(M)
    xs = {name: gen() for name, gen in acts.items()}
    ws = [(lin, oracle.binarize(lin.w())[0]) for lin in lins]   # weights are packed offline
    threads = max(1, min(16, os.cpu_count() or 1))

    def leg(n, thr):
        t0 = time.perf_counter()
        ts = {name: oracle.ternarize(x[:n])[0] for name, x in xs.items()}
        t1 = time.perf_counter()
        ops = 0.0
        for lin, s in ws:
            oracle.matmul_i32(ts[inputs.LLAMA7B_INPUTS[lin.name]], s, threads=thr)
            ops += 2.0 * n * lin.N * lin.K
        t2 = time.perf_counter()
        return t1 - t0, t2 - t1, ops
    tern_s, gemm_s, ops = leg(rows, threads)
    tern1, gemm1, ops1 = leg(rows_1t, 1)
    scale = rows / rows_1t
    dt = tern_s + gemm_s
    return {"value": round(ops / dt / 1e12, 4), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "cpu_model": _cpu_model(), "seconds": round(dt, 2),
            "ternarize_s": round(tern_s, 3), "gemm_s": round(gemm_s, 2),
            "sample": f"ternarize + dense int32 product of the first {rows} of {M} token rows "
                      f"of all seven LLaMA-7B layer GEMMs ({ops / 1e9:.0f} G ops), {threads} threads",
            "one_thread": {"rows": rows_1t, "extrapolated_to_rows": rows,
                           "ternarize_s": round(tern1 * scale, 2),
                           "gemm_s": round(gemm1 * scale, 1),
                           "value": round(ops1 / (tern1 + gemm1) / 1e12, 5), "unit": "TOPS"}}


def calibrate_copy(nbytes=256 << 20, reps=3):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE, WRITE_SIZE) of a profiler run."""
    import torch
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def profile_gemv(bw, copies=4):
    """A few cold launches of each decode shape, of gate/up stacked into one
    [57344, 8192] weight, and of the fused decode call (bf16 rows in, the
    shared workspace) for profiler counters."""
    import torch
    from binary_ternary_matmul_amd import inputs
    up = None
    for M in (1, 4, 16):
        for lin in inputs.llama70b_decode(M):
            w = bw.bwta_pack_weights(dev(lin.w()))
            ws = [w] + [bw.BinaryPlanes(w.sign.clone(), w.alpha.clone(), w.K) for _ in range(copies - 1)]
            a = bw.bwta_ternarize_pack(dev(lin.x()))
            y = torch.empty((M, lin.N), dtype=torch.float32, device="cuda")
            torch.cuda.synchronize()
            for wi in ws:
                bw.bwta_gemv(a, wi, "f32", "auto", y)
            torch.cuda.synchronize()
            if lin.name == "gate_up":  # then gate and up stacked, one launch
                if up is None:
                    up = bw.bwta_pack_weights(dev(inputs.llama70b_up_weight()()))
                fs = [bw.BinaryPlanes(torch.cat([g.sign, up.sign]), torch.cat([g.alpha, up.alpha]), g.K)
                      for g in ws]
                y2 = torch.empty((M, 2 * lin.N), dtype=torch.float32, device="cuda")
                torch.cuda.synchronize()
                for wi in fs:
                    bw.bwta_gemv(a, wi, "f32", "auto", y2)
                torch.cuda.synchronize()
                del fs
            X = dev(lin.x())  # the decode linear in one launch, bf16 rows in
            bw.bwta_gemv_fused(X, ws[0], "f32", y)  # (sizes the shared workspace)
            torch.cuda.synchronize()
            for wi in ws:
                bw.bwta_gemv_fused(X, wi, "f32", y)
            torch.cuda.synchronize()
            del ws, w
    print(json.dumps({"profile_gemv": "done", "copies": copies}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--quick", action="store_true", help="prefill step only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 256 MiB device copy (profiler byte-counter scale)")
    ap.add_argument("--profile-gemv", action="store_true",
                    help="only run a few cold launches of each decode GEMV shape")
    ap.add_argument("--attention", action="store_true",
                    help="only the attention section (unfused products and the fused call)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only the measured ceilings (HBM read streams, MFMA loops)")
    ap.add_argument("--gemv", action="store_true",
                    help="only the decode section (GEMV shapes and the decode linear end to end)")
    ap.add_argument("--bert", action="store_true",
                    help="only the BERT-base encoder linears (ternarize + product each)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return
    import binary_ternary_matmul_amd as bw
    bw.lib()
    if args.profile_gemv:
        profile_gemv(bw)
        return
    if args.attention:
        print(json.dumps({"attention": bench_attention(bw)}), flush=True)
        return
    if args.ceilings:
        print(json.dumps({"ceilings": ceilings()}), flush=True)
        return
    if args.gemv:
        print(json.dumps({"gemv": bench_gemv(bw)}), flush=True)
        return
    if args.bert:
        print(json.dumps({"bert": bench_bert(bw)}), flush=True)
        return

    from binary_ternary_matmul_amd import inputs
    pre = bench_prefill(bw, args.steps, args.warmup)
    achieved = pre["ops"] / (pre["gemm_ms"] * 1e-3) / 1e12
    line = {
        "metric": "binary×ternary GEMM TOPS (% int8 MFMA peak); decode GEMV HBM GB/s",
        "value": round(pre["ops"] / (pre["ms_step"] * 1e-3) / 1e12, 1),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4",
        "data": "synthetic",
        "config": {"workload": "llama7b_prefill_layer_linears", "tokens": pre["M"],
                   "gemms": {k: [v["M"], v["N"], v["K"]] for k, v in pre["per_gemm"].items()},
                   "stacked": {name: list(parts) for name, parts in inputs.LLAMA7B_PRODUCTS
                               if len(parts) > 1},
                   "activations": "bf16 Student-t(3), 1% outlier channels x50",
                   "weights": "N(0,0.02) packed to 1 bit", "out": "bf16",
                   "ops_per_step": pre["ops"]},
        "gemm_frac_of_int8_peak": round(achieved / INT8_PEAK_TOPS, 3),
        "ternarize_us_per_step": round(pre["ternarize_ms"] * 1e3, 1),
        "ternarize_roofline": pre["ternarize_roofline"],
        "host_wall_ms_per_step": round(pre["wall_ms_step"], 4),
        "per_gemm": pre["per_gemm"],
        "roofline": {"bound": "mfma", "kernel": "gemm_mfma_kernel", "achieved": round(achieved, 1),
                     "peak": FP4_PEAK_TOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / FP4_PEAK_TOPS, 3), "traffic": None},
    }
    tr = profiled_traffic("gemm_mfma_kernel")
    if tr:
        line["roofline"]["traffic"] = tr["bytes"]
        line["roofline"]["traffic_algorithmic"] = tr["algorithmic_bytes"]
        line["roofline"]["traffic_source"] = tr["summary"]
    if not args.quick:
        log("[bench] ceilings (probe kernels)")
        line["ceilings"] = ceilings()
        # the ternarize inputs' bytes through the pure read stream, for scale
        for name, x in pre["X"].items():
            t = line["ternarize_roofline"]["per_input"][name]
            t["read_probe_us"] = round(probe_read_us(x), 2)
            t["time_vs_read_probe"] = round(t["us"] / t["read_probe_us"], 2)
        fp4_loop = line["ceilings"]["fp4_mfma_loop_TOPS"]
        line["roofline"]["measured_peak"] = fp4_loop
        line["roofline"]["frac_of_measured_peak"] = round(achieved / fp4_loop, 3)
        log("[bench] int8 MFMA variant")
        line["mfma_i8"] = bench_algo(bw, pre, "mfma_i8")
        log("[bench] popcount variant")
        line["popcount"] = bench_algo(bw, pre, "popcount")
        log("[bench] two-plane residual weights")
        line["residual"] = bench_residual(bw, pre)
        log("[bench] gemv")
        line["gemv"] = bench_gemv(bw)
        if "roofline" in line["gemv"]:
            # the long stream: the short one (one decode weight per launch) measures
            # below what the decode kernels themselves reach
            hb = line["ceilings"]["hbm_read_1GiB_GBps"]
            line["gemv"]["roofline"]["measured_peak"] = hb
            line["gemv"]["roofline"]["frac_of_measured_peak"] = round(
                line["gemv"]["roofline"]["achieved"] / hb, 3)
        log("[bench] gemv, two-plane residual weights")
        line["residual"]["decode"] = bench_gemv_residual(bw)
        log("[bench] attention")
        line["attention"] = bench_attention(bw)
        log("[bench] bert")
        line["bert"] = bench_bert(bw)
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
