#!/usr/bin/env python3
"""Benchmark of the W8A8 block-scaled FP8 projection on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload large_prefill]

One step = one pass of the whole projection over one batch of synthetic
input, already resident in HBM: activation quantizer -> scale relayout ->
block-scaled FP8 GEMM (the calls fp8q_proj makes, issued separately so the
GEMM can be bracketed by events; for small batches the quantizer writes the
K-major scales itself, as fp8q_proj does).

Default workload: the large prefill projection M=4576, K=17408, N=5120,
Laplace(0,1) activations with 0.5% outlier channels x50, weights N(0,0.02)
quantized per 128x128 block.  Prints ONE JSON line:

  value           whole-step TFLOP/s = 2*M*N*K / step time
  roofline        the GEMM (dominant kernel) against the dense FP8 MFMA peak
                  (HBM peak for the skinny decode kernel), duration from HIP
                  events around each GEMM launch of the timed steps; also
                  R back-to-back launches between two events (no host gaps)
  act_quant       the quantizer's GB/s (algorithmic bytes) against HBM peak
  cpu_baseline    the CPU oracle on a bounded sample of the same workload
  bf16_comparator the same GEMM in bf16 over the dequantized weights (our
                  bf16 MFMA kernel and hipBLASLt), and the FP8 speedup
  fp8_library_comparator  hipBLASLt's FP8 GEMM (torch._scaled_mm) on the same
                  codes with per-tensor / per-row scales, for context

Other modes (one JSON line each, not the benchmark line): --quant-sweep,
--dequant, --ffn <workload> (the dense FFN chain), --ffn-sweep (its
selector), --gemm-sweep (split-K), --cpu-sweep (the CPU oracle baseline
per shape), --copy-mib N.

Only one GPU is used; --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA, TFLOP/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
# HBM bytes the rocprofv3 FETCH_SIZE/WRITE_SIZE counters attribute to one
# launch of the dominant GEMM at the default workload, scaled by the counters'
# readings for a plain 1 GiB copy (the HBM-bytes summary under profiles/).
# Valid only for the kernel source they were taken with: reported as null
# once the ping-pong kernel's source changes (gemm_source_hash).
GEMM_TRAFFIC = {"bytes": 1.2274e+09 + 4.7088e+07, "gemm_source_sha256": "e3d4b625424f3c35"}


def gemm_source_hash():
    """SHA-256 prefix of the ping-pong kernel's source (its section of
    gemm.hip, from its header comment to the skinny kernel's, and the shared
    tile helpers): the traffic figure stays valid while these are unchanged."""
    import hashlib
    csrc = os.path.join(ROOT, "w8a8_fp8_block_amd", "csrc")
    g = open(os.path.join(csrc, "gemm.hip")).read()
    i, j = g.index("// Ping-pong kernel:"), g.index("// Skinny kernel for decode")
    text = g[i:j] + open(os.path.join(csrc, "mfma_common.h")).read()
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def gemm_traffic():
    return GEMM_TRAFFIC["bytes"] if gemm_source_hash() == GEMM_TRAFFIC["gemm_source_sha256"] else None


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="large_prefill",
                   choices=["tiny", "decode", "prefill", "large_prefill"])
    p.add_argument("--M", type=int, default=None, help="row count for the decode sweep")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="approximate CPU time budget of the oracle sample")
    p.add_argument("--weights", default="block", choices=["block", "row"],
                   help="FP8 weight scales: one per 128x128 block (default) or one per row")
    p.add_argument("--dequant", action="store_true",
                   help="instead of the benchmark, time the FP8 -> bf16 weight dequantizer on "
                        "the prefill and large-prefill weights, both scale formats")
    p.add_argument("--quant-sweep", action="store_true",
                   help="instead of the benchmark, time quantizer variants A, B and the "
                        "selector's choice over the token/K sweep (one JSON line per shape)")
    p.add_argument("--ffn", default=None, choices=["ffn_decode", "ffn_prefill", "ffn_large"],
                   help="time the dense FFN chain (fp8q_ffn, both variants, and its kernels) "
                        "on this workload instead of the projection")
    p.add_argument("--ffn-sweep", action="store_true",
                   help="fp8q_ffn's two variants over M at H=5120, I=17408 with cold caches, "
                        "and the automatic choice (the selector's measurement)")
    p.add_argument("--gemm-sweep", action="store_true",
                   help="the GEMM's single-pass kernels and split-K counts over M at three "
                        "projection shapes with cold caches (the split-K selector's measurement)")
    p.add_argument("--cpu-sweep", action="store_true",
                   help="instead of the benchmark, time the CPU oracle on the host cores: "
                        "quantizer + relayout per quantizer-sweep shape (all threads and one), "
                        "fp64 GEMM per GEMM workload (no GPU used)")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="instead of the benchmark, run 3 plain device copies of this many "
                        "MiB (the reference kernel for scaling rocprofv3 byte counters)")
    return p.parse_args()


def copy_calibration(mib: int):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def quant_sweep(reps=25):
    """Quantizer variants A and B and the automatic choice on every (M, K) of
    the token/K sweep plus M in {17, 64, 128, 256, 512}: median kernel time
    over `reps` launches, each after a 1 GiB write that evicts L2 and the
    256 MB last-level cache, plus the selection rule check
    t(auto) <= 1.03 * min(t_A, t_B) + 0.1 us."""
    import torch
    import synth
    import w8a8_fp8_block_amd as fp8q
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sweep = synth.WORKLOADS["quant_sweep"]
    Ks = sorted({w.K for w in sweep})
    Ms = sorted({w.M for w in sweep} | {17, 64, 128, 256, 512})
    for K in Ks:
        G = K // 128
        base = next(w for w in sweep if w.K == K)
        for M in Ms:
            x = torch.from_numpy(synth.make_inputs(base, M=M, with_weights=False)[0]
                                 .view(np.int16)).to(dev)
            q = torch.empty((M, K), dtype=torch.uint8, device=dev)
            sc = torch.empty((M, G), dtype=torch.float32, device=dev)
            times = {}
            for name, var in (("A", 1), ("B", 2), ("auto", 0)):
                ts = []
                for _ in range(reps):
                    flush.fill_(1)
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    fp8q.fp8q_quant_act(x, q, sc, variant=var)
                    e1.record()
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1) * 1e3)
                times[name] = float(np.median(ts))
            v, grid, why = fp8q.fp8q_quant_select(M, K, cus)
            nbytes = 3 * M * K + 4 * M * G
            best = min(times["A"], times["B"])
            print(json.dumps({
                "M": M, "K": K, "t_A_us": round(times["A"], 2), "t_B_us": round(times["B"], 2),
                "t_auto_us": round(times["auto"], 2), "auto": "B" if v == 2 else "A",
                "grid_B": (M * ((G + 31) // 32)), "reject": why,
                "best_GBs": round(nbytes / best / 1e3, 1),
                "best_frac_hbm": round(nbytes / best / 1e3 / HBM_PEAK_GBS, 4),
                "rule_ok": times["auto"] <= 1.03 * best + 0.1}), flush=True)


def dequant_bench(reps=20):
    """FP8 -> bf16 weight expansion (HBM-bound: 1 byte read, 2 written per
    element) on the prefill (N=17408, K=5120) and large-prefill (N=5120,
    K=17408) weights, block-scaled and per-row, two weight copies alternated
    so successive launches do not hit the cache."""
    import torch
    import synth
    import w8a8_fp8_block_amd as fp8q
    dev = torch.device("cuda:0")
    for name in ("prefill", "large_prefill"):
        w = synth.WORKLOADS[name][0]
        _, wf, _ = synth.make_inputs(w, M=1)
        wf = torch.from_numpy(wf).to(dev)
        for per_row in (False, True):
            codes, sc = quantize_weights_gpu(wf, per_row)
            copies = [(codes, sc), (codes.clone(), sc.clone())]
            dst = torch.empty((w.N, w.K), dtype=torch.bfloat16, device=dev)
            for c, s_ in copies:
                fp8q.fp8q_dequant_fp8_bf16(c, s_, dst, per_row)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                c, s_ = copies[i % 2]
                fp8q.fp8q_dequant_fp8_bf16(c, s_, dst, per_row)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            nbytes = 3 * w.N * w.K + 4 * sc.numel()
            print(json.dumps({"dequant": f"{name} N={w.N} K={w.K}",
                              "scales": "per-row" if per_row else "128x128 blocks",
                              "us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1),
                              "frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}), flush=True)


def ffn_bench(name: str, M=None, reps=20):
    """The dense FFN chain x[M,H] -> gate, up [I,H] -> SiLU * up -> down [H,I]
    (fp8q_ffn) on one synthetic workload: the whole call for both variants
    (median with the caches flushed before each call, and back to back), and
    its kernels one by one (R back-to-back launches between two events):
    the input quantizer, the fused gate/up kernel, the separate path's two
    GEMMs and fp8q_silu_mul_quant, and the down GEMM.  FLOPs: 2*M*H*I per
    projection, three projections."""
    import torch
    import synth
    import w8a8_fp8_block_amd as fp8q
    dev = torch.device("cuda:0")
    w = synth.ffn_workload(name, M)
    M, H, I = w.M, w.H, w.I
    print(f"[bench] ffn inputs {w.desc}", file=sys.stderr, flush=True)
    xb, (wg, wu, wd) = synth.make_ffn_inputs(w)
    x = torch.from_numpy(xb.view(np.int16)).to(dev)
    (gq, gs), (uq, us), (dq, ds) = (quantize_weights_gpu(torch.from_numpy(a).to(dev))
                                    for a in (wg, wu, wd))
    del wg, wu, wd
    out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    ws = {v: fp8q.alloc_ffn_workspace(M, H, I, v) for v in (1, 2)}

    def timed(fn, n=reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def timed_cold(fn, n=reps):
        """median over n calls, each after a 512 MiB write that evicts L2 and
        the 256 MB last-level cache (one layer's weights are not resident)"""
        fn()
        ts = []
        for _ in range(n):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    flops = 6.0 * M * H * I
    res = {"ffn": w.desc, "auto_variant": fp8q.fp8q_ffn_select(M, H, I)}
    fns = {v: (lambda v=v: fp8q.fp8q_ffn(x, gq, gs, uq, us, dq, ds, out, ws[v], variant=v))
           for v in (1, 2)}
    cold = {1: [], 2: []}
    for r in range(2 * reps + 2):  # alternating, so clock drift hits both variants
        v = 1 + (r & 1)
        t1 = timed_cold(fns[v], n=1)
        if r >= 2:
            cold[v].append(t1)
    for v in (1, 2):
        us_ = float(np.median(cold[v]))
        res[f"variant{v}_cold_us"] = round(us_, 2)
        res[f"variant{v}_cold_tflops"] = round(flops / us_ / 1e6, 1)
        res[f"variant{v}_back_to_back_us"] = round(timed(fns[v]), 2)
    # the pieces
    Mp = fp8q.fp8q_m_pad(M)
    xq = torch.empty((M, H), dtype=torch.uint8, device=dev)
    xs = torch.empty((M, H // 128), dtype=torch.float32, device=dev)
    xkm = torch.empty((H // 128, Mp), dtype=torch.float32, device=dev)
    fp8q.fp8q_quant_act_kmajor(x, xq, xs, xkm)
    hq = torch.empty((M, I), dtype=torch.uint8, device=dev)
    hkm = torch.empty((I // 128, Mp), dtype=torch.float32, device=dev)
    g = torch.empty((M, I), dtype=torch.bfloat16, device=dev)
    u = torch.empty((M, I), dtype=torch.bfloat16, device=dev)
    res["quant_x_us"] = round(timed(lambda: fp8q.fp8q_quant_act_kmajor(x, xq, xs, xkm)), 2)
    t = timed(lambda: fp8q.fp8q_ffn_gate_up(xq, xkm, gq, gs, uq, us, hq, hkm))
    res["gate_up_fused_us"] = round(t, 2)
    res["gate_up_fused_tflops"] = round(4.0 * M * H * I / t / 1e6, 1)
    res["gate_up_fused_frac_fp8_peak"] = round(4.0 * M * H * I / t / 1e6 / FP8_PEAK_TFLOPS, 4)
    res["gate_gemm_us"] = round(timed(lambda: fp8q.fp8q_gemm_blockscaled(xq, xkm, gq, gs, g)), 2)
    res["up_gemm_us"] = round(timed(lambda: fp8q.fp8q_gemm_blockscaled(xq, xkm, uq, us, u)), 2)
    t = timed(lambda: fp8q.fp8q_silu_mul_quant(g, u, hq, hkm))
    nbytes = 4 * M * I + M * I + 4 * Mp * (I // 128)
    res["silu_mul_quant_us"] = round(t, 2)
    res["silu_mul_quant_frac_hbm"] = round(nbytes / t / 1e3 / HBM_PEAK_GBS, 4)
    fp8q.fp8q_ffn_gate_up(xq, xkm, gq, gs, uq, us, hq, hkm)
    res["down_gemm_us"] = round(timed(lambda: fp8q.fp8q_gemm_blockscaled(hq, hkm, dq, ds, out)), 2)
    res["down_kernel"] = fp8q.GEMM_KERNEL_NAMES[fp8q.fp8q_gemm_select(M, H, I)]
    print(json.dumps(res), flush=True)


def ffn_sweep(reps=15):
    """fp8q_ffn variants 1 (fused gate/up) and 2 (separate) over M at H=5120,
    I=17408: median time of the whole call over `reps` calls of each, the
    two variants alternating, each call after a 512 MiB write that evicts L2
    and the last-level cache; and whether the automatic choice is within 3%
    of the faster variant."""
    import torch
    import synth
    import w8a8_fp8_block_amd as fp8q
    dev = torch.device("cuda:0")
    base = synth.ffn_workload("ffn_prefill")
    H, I = base.H, base.I
    _, (wg, wu, wd) = synth.make_ffn_inputs(base, M=1)
    (gq, gs), (uq, us), (dq, ds) = (quantize_weights_gpu(torch.from_numpy(a).to(dev))
                                    for a in (wg, wu, wd))
    del wg, wu, wd
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for M in (16, 25, 32, 33, 48, 64, 80, 128, 256, 512, 1168, 2048, 4576):
        xb, _ = synth.make_ffn_inputs(base, M=M, with_weights=False)
        x = torch.from_numpy(xb.view(np.int16)).to(dev)
        out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        ws = {v: fp8q.alloc_ffn_workspace(M, H, I, v) for v in (1, 2)}
        ts = {1: [], 2: []}
        for r in range(2 * reps):  # the variants alternate: clock drift hits both
            v = 1 + (r & 1)
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fp8q.fp8q_ffn(x, gq, gs, uq, us, dq, ds, out, ws[v], variant=v)
            e1.record()
            torch.cuda.synchronize()
            if r >= 2:
                ts[v].append(e0.elapsed_time(e1) * 1e3)
        t = {v: float(np.median(ts[v])) for v in (1, 2)}
        del ws
        auto = fp8q.fp8q_ffn_select(M, H, I)
        print(json.dumps({"M": M, "H": H, "I": I, "fused_us": round(t[1], 1),
                          "separate_us": round(t[2], 1), "auto": "fused" if auto == 1 else "separate",
                          "auto_tflops": round(6.0 * M * H * I / t[auto] / 1e6, 1),
                          "rule_ok": t[auto] <= 1.03 * min(t[1], t[2])}), flush=True)


def gemm_sweep(reps=10):
    """The block-scaled GEMM over M at three projection shapes, cold caches:
    the automatic single-pass kernel, the 128x128 tiled kernel and its split-K
    form at 2..12 splits (median of `reps` calls each, all variants taking turns,
    each call after a 512 MiB write that evicts L2 and the last-level cache);
    and whether fp8q_gemm_blockscaled_splitk's automatic choice is within 3% of
    the fastest variant.  Normal activations, quantized by the library;
    weights normal(0, 0.02), block-quantized."""
    import torch
    import w8a8_fp8_block_amd as fp8q
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for N, K in ((5120, 17408), (6144, 5120), (17408, 5120)):
        wq, wsc = quantize_weights_gpu(torch.randn((N, K), generator=gen, device=dev) * 0.02)
        for M in (16, 32, 64, 65, 96, 128, 192, 256, 384, 512, 768, 1024, 1168, 1536, 2048):
            x = torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16)
            q = torch.empty((M, K), dtype=torch.uint8, device=dev)
            srm = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
            skm = torch.empty((K // 128, fp8q.fp8q_m_pad(M)), dtype=torch.float32, device=dev)
            fp8q.fp8q_quant_act_kmajor(x, q, srm, skm)
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            auto_k = fp8q.fp8q_gemm_select(M, N, K)
            variants = {"auto": ("k", 0), "k1": ("k", 1)}
            for S in (2, 3, 4, 6, 8, 12):
                variants[f"s{S}"] = ("s", S)
            wsp = torch.empty((12 * M * N,), dtype=torch.float32, device=dev)
            names = list(variants)
            ts = {v: [] for v in names}
            for r in range(reps + 1):
                for v in names:
                    kind, arg = variants[v]
                    flush.fill_(1)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    if kind == "k":
                        fp8q.fp8q_gemm_blockscaled(q, skm, wq, wsc, out, kernel=arg)
                    else:
                        fp8q.fp8q_gemm_blockscaled_splitk(q, skm, wq, wsc, out, wsp, splits=arg)
                    e1.record()
                    torch.cuda.synchronize()
                    if r >= 1:
                        ts[v].append(e0.elapsed_time(e1) * 1e3)
            t = {v: round(float(np.median(ts[v])), 1) for v in names}
            best = min(t, key=t.get)
            sel = fp8q.fp8q_gemm_splitk_select(M, N, K)
            chosen = t["auto"] if sel < 2 else t[f"s{sel}"] if f"s{sel}" in t else None
            print(json.dumps({"M": M, "N": N, "K": K, "auto_kernel": auto_k, "us": t,
                              "best": best, "splitk_auto": sel,
                              "rule_ok": None if chosen is None else chosen <= 1.03 * t[best]}),
                  flush=True)
            del wsp, x, q, srm, skm, out
        del wq, wsc


def cpu_sweep():
    """The oracle on the host cores, as the CPU baseline plan lays out: the
    quantizer + relayout on every quantizer-sweep shape (all threads and one
    thread) and the fp64 block GEMM on every GEMM workload; the median of 3
    runs (one run where a run exceeds 30 s).  One JSON line per item."""
    import ctypes
    import oracle
    import synth
    oracle._load()
    threads = oracle.num_threads()
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    gomp = ctypes.CDLL("libgomp.so.1")

    def med3(fn):
        t0 = time.perf_counter()
        fn()
        t = [time.perf_counter() - t0]
        if t[0] <= 30.0:
            for _ in range(2):
                t0 = time.perf_counter()
                fn()
                t.append(time.perf_counter() - t0)
        return float(np.median(t)), len(t)

    print(json.dumps({"cpu_model": model, "threads": threads}), flush=True)
    for w in synth.WORKLOADS["quant_sweep"]:
        x, _, _ = synth.make_inputs(w)
        nbytes = w.M * w.K * 2 + w.M * w.K + w.M * (w.K // 128) * 4      # quantizer
        nbytes += w.M * (w.K // 128) * 4 + synth.ceil16(w.M) * (w.K // 128) * 4  # relayout

        def q():
            _, a_s = oracle.quant_act(x)
            oracle.scale_to_kmajor(a_s)
        t, n = med3(q)
        gomp.omp_set_num_threads(1)
        try:
            t1, n1 = med3(q)
        finally:
            gomp.omp_set_num_threads(threads)
        print(json.dumps({"item": "quant+relayout", "M": w.M, "K": w.K, "s": round(t, 5),
                          "GBps": round(nbytes / t / 1e9, 2), "runs": n,
                          "s_1thread": round(t1, 5), "GBps_1thread": round(nbytes / t1 / 1e9, 3)}),
              flush=True)
        del x
    for name in ("tiny", "decode", "prefill", "large_prefill"):
        for w in synth.WORKLOADS[name]:
            x, wf, _ = synth.make_inputs(w)
            a, a_s = oracle.quant_act(x)
            wq, ws = oracle.quant_weight_block(wf)
            del wf
            t, n = med3(lambda: oracle.gemm_ref(a, a_s, wq, ws))
            print(json.dumps({"item": "fp64 block GEMM", "workload": w.desc, "s": round(t, 4),
                              "GFLOPs": round(2.0 * w.M * w.N * w.K / t / 1e9, 2), "runs": n}),
                  flush=True)
            del x, a, wq


def quantize_weights_gpu(wf, per_row=False):
    """Synthetic FP8 weights: per 128x128 block (or per row), scale = amax/448,
    codes by PyTorch's float8_e4m3fn cast (input preparation, outside the timed
    path)."""
    import torch
    N, K = wf.shape
    if per_row:
        ws = (wf.abs().amax(dim=1) / 448.0).to(torch.float32)
        safe = torch.where(ws > 0, ws, torch.ones_like(ws))
        q = (wf / safe[:, None]).clamp(-448, 448)
        return q.to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), ws.contiguous()
    blocks = wf.view(N // 128, 128, K // 128, 128)
    amax = blocks.abs().amax(dim=(1, 3))
    ws = (amax / 448.0).to(torch.float32)
    safe = torch.where(ws > 0, ws, torch.ones_like(ws))
    q = (blocks / safe[:, None, :, None]).clamp(-448, 448)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(N, K).contiguous()
    return codes, ws.contiguous()


def cpu_baseline(w, x_bits, wf, budget_s, per_row=False):
    """Time the oracle (quantizer + relayout + fp64 GEMM) on the first R rows."""
    import oracle
    oracle._load()
    # input preparation, not timed
    wq, ws = oracle.quant_weight_row(wf) if per_row else oracle.quant_weight_block(wf)
    threads = oracle.num_threads()
    # calibrate on 2 rows, then size the sample to the budget
    def run(R):
        xs = np.ascontiguousarray(x_bits[:R])
        t0 = time.perf_counter()
        a, a_s = oracle.quant_act(xs)
        oracle.scale_to_kmajor(a_s)
        t1 = time.perf_counter()
        oracle.gemm_ref(a, a_s, wq, ws)
        return t1 - t0, time.perf_counter() - t1
    t2 = sum(run(2))
    R = int(max(2, min(w.M, 2 * budget_s / max(t2, 1e-6))))
    R = max(2, min(R, w.M))
    tq, tg = run(R)
    t = tq + tg
    # the quantizer and relayout on one thread as well (OpenMP runtime of the oracle)
    tq1 = None
    try:
        import ctypes
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        try:
            xs = np.ascontiguousarray(x_bits[:R])
            t0 = time.perf_counter()
            _, a_s = oracle.quant_act(xs)
            oracle.scale_to_kmajor(a_s)
            tq1 = time.perf_counter() - t0
        finally:
            gomp.omp_set_num_threads(threads)
    except OSError:
        pass
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    flops = 2.0 * R * w.N * w.K
    return {
        "value": round(flops / t / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {R} of {w.M} rows of {w.desc}: quantize + relayout + fp64 block GEMM "
                  f"({t:.1f} s, one run)",
        "cpu_model": model,
        "quant_relayout_s": round(tq, 4),
        "gemm_s": round(tg, 3),
        "quant_relayout_1thread_s": None if tq1 is None else round(tq1, 4),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the projection runs on exactly one GPU here; --gpus {args.gpus} is "
              "not supported (one GPU's share is the workload; multi-GPU sharding is not built)",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_mib:
        copy_calibration(args.copy_mib)
        return
    if args.cpu_sweep:
        cpu_sweep()
        return
    if args.quant_sweep:
        quant_sweep()
        return
    if args.dequant:
        dequant_bench()
        return
    if args.ffn:
        ffn_bench(args.ffn, args.M)
        return
    if args.ffn_sweep:
        ffn_sweep()
        return
    if args.gemm_sweep:
        gemm_sweep()
        return

    import torch
    import synth
    import w8a8_fp8_block_amd as fp8q

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)

    w = (synth.workload(args.workload, M=args.M) if args.workload == "decode"
         else synth.workload(args.workload))
    M, K, N = w.M, w.K, w.N
    G = K // 128
    print(f"[bench] inputs {w.desc} (seed {w.seed})", file=sys.stderr, flush=True)
    x_bits, wf, _ = synth.make_inputs(w)
    x = torch.from_numpy(x_bits.view(np.int16)).to(dev)
    per_row = args.weights == "row"
    wq, ws = quantize_weights_gpu(torch.from_numpy(wf).to(dev), per_row)
    gemm = fp8q.fp8q_gemm_rowscaled if per_row else fp8q.fp8q_gemm_blockscaled
    act_q, act_s, act_km = fp8q.alloc_proj_scratch(M, K)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    variant, grid, why = fp8q.fp8q_quant_select(M, K, props.multi_processor_count)

    fused = fp8q.fp8q_proj_quant_fused(M, K)  # the same choice fp8q_proj makes

    def step(ev_q=None, ev_g=None):
        if ev_q: ev_q[0].record(stream)
        if fused:
            fp8q.fp8q_quant_act_kmajor(x, act_q, act_s, act_km)
        else:
            fp8q.fp8q_quant_act(x, act_q, act_s)
        if ev_q: ev_q[1].record(stream)
        if not fused:
            fp8q.fp8q_scale_to_kmajor(act_s, act_km)
        if ev_g: ev_g[0].record(stream)
        gemm(act_q, act_km, wq, ws, out)
        if ev_g: ev_g[1].record(stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evq = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    evg = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(evq[i], evg[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    # Back-to-back kernel timings: R launches of one kernel between two events
    # (no host gaps inside; at decode widths the Python-driven step above is
    # host-launch-bound and its per-launch events include those gaps).  The
    # GEMM alternates between two weight copies when they fit, so its weight
    # stream is not served from the previous launch's cache lines.
    R = 20
    w_alt = [wq]
    if N * K <= (1 << 30):
        w_alt.append(wq.clone())
    x_alt = [x, x.clone()] if M * K * 2 <= (1 << 30) else [x]
    torch.cuda.synchronize()
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for i in range(R):
        gemm(act_q, act_km, w_alt[i % len(w_alt)], ws, out)
    b1.record(stream)
    torch.cuda.synchronize()
    gemm_b2b_us = b0.elapsed_time(b1) * 1e3 / R
    b0.record(stream)
    for i in range(R):
        fp8q.fp8q_quant_act(x_alt[i % len(x_alt)], act_q, act_s)
    b1.record(stream)
    torch.cuda.synchronize()
    quant_b2b_us = b0.elapsed_time(b1) * 1e3 / R
    del w_alt, x_alt

    # bf16 comparator: the same projection in bf16 over the weights
    # dequantized once by fp8q_dequant_fp8_bf16 (outside the timing); our bf16
    # MFMA kernel and, for context, the vendor library through torch.mm
    # (hipBLASLt), each R back-to-back launches alternating two weight copies
    wd = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    fp8q.fp8q_dequant_fp8_bf16(wq, ws, wd, per_row)
    xb = x.view(torch.bfloat16)
    outb = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    wds = [wd, wd.clone()]
    torch.cuda.synchronize()
    b0.record(stream)
    for i in range(R):
        fp8q.fp8q_gemm_bf16(xb, wds[i % 2], outb)
    b1.record(stream)
    torch.cuda.synchronize()
    bf16_own_us = b0.elapsed_time(b1) * 1e3 / R
    wts = [t.t().contiguous() for t in wds]  # [K,N] for a plain (non-batched) mm
    del wds
    torch.mm(xb, wts[0], out=outb)
    torch.cuda.synchronize()
    b0.record(stream)
    for i in range(R):
        torch.mm(xb, wts[i % 2], out=outb)
    b1.record(stream)
    torch.cuda.synchronize()
    bf16_lib_us = b0.elapsed_time(b1) * 1e3 / R
    del wts, wd

    # FP8 library comparator (context): the vendor library's FP8 GEMM through
    # torch._scaled_mm on the same code bytes, with the scaling modes it
    # offers (one scale per tensor; one per activation row and weight row)
    # instead of 128x128 blocks -- a different, simpler operation
    fp8_lib = {}
    if not per_row and hasattr(torch, "_scaled_mm"):
        a8 = act_q.view(torch.float8_e4m3fn)
        w8s = [wq.view(torch.float8_e4m3fn), wq.clone().view(torch.float8_e4m3fn)]
        one = torch.ones((), dtype=torch.float32, device=dev)
        modes = {"per_tensor": (one, one),
                 "rowwise": (torch.ones((M, 1), dtype=torch.float32, device=dev),
                             torch.ones((1, N), dtype=torch.float32, device=dev))}
        for name, (sa, sb) in modes.items():
            try:
                torch._scaled_mm(a8, w8s[0].t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
                torch.cuda.synchronize()
                b0.record(stream)
                for i in range(R):
                    torch._scaled_mm(a8, w8s[i % 2].t(), scale_a=sa, scale_b=sb,
                                     out_dtype=torch.bfloat16)
                b1.record(stream)
                torch.cuda.synchronize()
                us = b0.elapsed_time(b1) * 1e3 / R
                fp8_lib[name] = {"us": round(us, 2), "tflops": round(2.0 * M * N * K / us / 1e6, 1)}
            except Exception as ex:  # not offered on this build / device
                fp8_lib[name] = {"error": str(ex).splitlines()[0][:160]}
        del w8s
    del outb

    gpu_ms = t_start.elapsed_time(t_end)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    gemm_ms = np.array([a.elapsed_time(b) for a, b in evg])
    quant_ms = np.array([a.elapsed_time(b) for a, b in evq])
    flops = 2.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_avg_s = float(np.mean(gemm_ms)) * 1e-3
    gemm_tflops = flops / gemm_avg_s / 1e12
    quant_bytes = M * K * 2 + M * K + M * G * 4
    quant_avg_s = float(np.mean(quant_ms)) * 1e-3
    quant_gbs = quant_bytes / quant_avg_s / 1e9

    def pct(ms):  # per-launch event times of the timed steps
        p10, p50, p90 = np.percentile(np.asarray(ms) * 1e3, [10, 50, 90])
        return {"p10_us": round(float(p10), 2), "median_us": round(float(p50), 2),
                "p90_us": round(float(p90), 2)}
    gemm_pct = pct(gemm_ms)

    kern = fp8q.fp8q_gemm_select(M, N, K)
    if kern == 2:
        # decode widths: the GEMM streams the weight matrix once (HBM-bound)
        gemm_bytes = N * K + M * K + 2 * M * N + 4 * (N // 128) * G + 4 * fp8q.fp8q_m_pad(M) * G
        gemm_gbs = gemm_bytes / gemm_avg_s / 1e9
        roofline = {"bound": "hbm", "kernel": fp8q.GEMM_KERNEL_NAMES[kern],
                    "achieved": round(gemm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gemm_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                    "avg_launch_us": round(gemm_avg_s * 1e6, 2),
                    **gemm_pct,
                    "back_to_back_us": round(gemm_b2b_us, 2),
                    "back_to_back_achieved": round(gemm_bytes / gemm_b2b_us / 1e3, 1),
                    "algorithmic_bytes_per_launch": gemm_bytes}
    else:
        roofline = {"bound": "mfma", "kernel": fp8q.GEMM_KERNEL_NAMES[kern],
                    "achieved": round(gemm_tflops, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(gemm_tflops / FP8_PEAK_TFLOPS, 4),
                    "traffic": (gemm_traffic() if args.workload == "large_prefill" and not per_row
                                else None),
                    "avg_launch_us": round(gemm_avg_s * 1e6, 2),
                    **gemm_pct,
                    "back_to_back_us": round(gemm_b2b_us, 2),
                    "back_to_back_achieved": round(flops / gemm_b2b_us / 1e6, 2),
                    "algorithmic_flops_per_launch": flops}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, x_bits, wf, args.cpu_seconds, per_row)

    rec = {
        "metric": "block-scaled FP8 proj TFLOP/s (M=4576) + act-quant GB/s vs HBM peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name} M={M} K={K} N={N}",
            "M": M, "K": K, "N": N,
            "activations": f"bf16 {w.dist}(0,1), {w.n_outliers} outlier channels x{w.outlier_factor:g}",
            "weights": ("fp8 e4m3 [N,K], fp32 scale per row (from N(0,0.02))" if per_row else
                        "fp8 e4m3 [N,K], fp32 scale per 128x128 block (from N(0,0.02))"),
            "output": "bf16 [M,N]",
            "step": (("act-quant writing both scale layouts" if fused else
                      "act-quant + scale relayout") +
                     (" + per-row-scaled FP8 GEMM" if per_row else " + block-scaled FP8 GEMM")),
            "quant_variant": "B" if variant == 2 else "A",
            "device": props.name, "gcn_arch": props.gcnArchName,
            "cus": props.multi_processor_count,
        },
        "roofline": roofline,
        "act_quant": {
            "achieved": round(quant_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(quant_gbs / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(quant_avg_s * 1e6, 2),
            **pct(quant_ms),
            "back_to_back_us": round(quant_b2b_us, 2),
            "back_to_back_achieved": round(quant_bytes / quant_b2b_us / 1e3, 1),
            "algorithmic_bytes_per_launch": quant_bytes,
        },
        "cpu_baseline": cpu,
        "bf16_comparator": {
            "what": "the same projection's GEMM in bf16 over the dequantized weights, "
                    "back-to-back launches",
            "own_bf16_us": round(bf16_own_us, 2),
            "own_bf16_tflops": round(flops / bf16_own_us / 1e6, 1),
            "hipblaslt_bf16_us": round(bf16_lib_us, 2),
            "hipblaslt_bf16_tflops": round(flops / bf16_lib_us / 1e6, 1),
            "fp8_back_to_back_us": round(gemm_b2b_us, 2),
            "fp8_over_own_bf16": round(bf16_own_us / gemm_b2b_us, 3),
            "fp8_over_hipblaslt_bf16": round(bf16_lib_us / gemm_b2b_us, 3),
            "bf16_peak_tflops": BF16_PEAK_TFLOPS,
        },
        "fp8_library_comparator": {
            "what": "hipBLASLt FP8 GEMM via torch._scaled_mm on the same code bytes with "
                    "per-tensor or per-row scales (not block scales), back-to-back launches",
            **fp8_lib,
        },
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
