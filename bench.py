#!/usr/bin/env python3
"""Benchmark of the W8A8 block-scaled FP8 projection on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload large_prefill]

One step = one pass of the whole projection over one batch of synthetic
input, already resident in HBM: activation quantizer -> scale relayout ->
block-scaled FP8 GEMM (the calls fp8q_proj makes, issued separately so that
each kernel can be bracketed by events; for small batches the quantizer
writes the K-major scales itself, as fp8q_proj does).  Before the W warmup
steps, untimed steps run for SETTLE_S seconds so that the device's power
control has settled (recorded as "settle" in each configuration).

Default workload: the large prefill projection M=4576, K=17408, N=5120,
Laplace(0,1) activations with 0.5% outlier channels x50, weights N(0,0.02)
quantized per 128x128 block.  Prints ONE JSON line:

  value           whole-step TFLOP/s = 2*M*N*K / step time (the timed steps'
                  span between two HIP events on the stream, over K;
                  timed_region also holds the host's wall time of it)
  roofline        the GEMM (dominant kernel) against the dense FP8 MFMA peak
                  (HBM peak for the weight-streaming skinny kernel): duration
                  from HIP events around each GEMM launch of the timed steps
                  (events without the system-scope fence, KernelEvents);
                  also R back-to-back launches between two events cycling
                  through weight copies of >= 600 MB (streamed from HBM, not
                  the 256 MB last-level cache), with the shader clock then
  act_quant       the quantizer's GB/s (algorithmic bytes) against HBM peak,
                  the same two ways
  clock           sustained shader clock over the timed steps, per XCD, from
                  clock stamps (fp8q_clock_stamp) before and after
  step_graph_us   the same step captured R times into one HIP graph and
                  replayed (no events, no host launches between kernels)
  cpu_baseline    the CPU oracle on a bounded sample of the same workload
  bf16_comparator the same GEMM in bf16 over the dequantized weights (our
                  bf16 MFMA kernel and hipBLASLt), and the FP8 speedup
  fp8_library_comparator  hipBLASLt's FP8 GEMM (torch._scaled_mm) on the same
                  codes with per-tensor / per-row scales, for context
  configs         the other workloads, each with its own step time, roofline,
                  act_quant, clock and oracle baseline: tiny (M=16, K=512,
                  N=256), decode_M16/17/25 (K=5120, N=6144), prefill
                  (M=1168, K=5120, N=17408) and quant_sweep (the 15
                  act-quant + scale-relayout shapes, M in {16, 25, 1168,
                  4576, 16384} x K in {5120, 6144, 17408})

Other modes (one JSON line each, not the benchmark line): --quant-sweep,
--dequant, --ffn <workload> (the dense FFN chain), --ffn-sweep (its
selector), --gemm-sweep (split-K, cold caches), --gemm-sweep-b2b (split-K up to
64 rows, back to back), --cpu-sweep (the CPU oracle baseline
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
# readings for a plain 64 MiB device copy (FETCH_SIZE x2, WRITE_SIZE x1;
# the HBM-bytes summary under profiles/).
# Valid only for the kernel source they were taken with: reported as null
# once the ping-pong kernel's source changes (gemm_source_hash).
GEMM_TRAFFIC = {"bytes": 1.2248e+09 + 4.7087e+07, "gemm_source_sha256": "ed4c14be68341a65"}


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
    p.add_argument("--only-workload", action="store_true",
                   help="time only --workload (skip the other configurations in the line)")
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
    p.add_argument("--gemm-sweep-b2b", action="store_true",
                   help="the GEMM's single pass and split-K counts up to 64 rows at three "
                        "projection shapes, back to back over rotating weight copies (the "
                        "split-K selector's measurement for those rows)")
    p.add_argument("--sweep-m", default=None,
                   help="comma-separated row counts for --gemm-sweep (default: its 15) or "
                        "--gemm-sweep-b2b (default: its 14)")
    p.add_argument("--cpu-sweep", action="store_true",
                   help="instead of the benchmark, time the CPU oracle on the host cores: "
                        "quantizer + relayout per quantizer-sweep shape (all threads and one), "
                        "fp64 GEMM per GEMM workload (no GPU used)")
    p.add_argument("--streamk-sweep", action="store_true",
                   help="instead of the benchmark, the stream-K GEMM against the single-pass "
                        "kernels at the shapes its automatic rule was fixed on")
    p.add_argument("--quant-vs-copy", action="store_true",
                   help="instead of the benchmark, the quantizer (variant A) and a plain device "
                        "copy of its input at the M >= 1168 sweep shapes, 20 launches each after "
                        "a 1 GiB read that evicts the caches (for a kernel trace)")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="instead of the benchmark, run 3 plain device copies of this many "
                        "MiB (the reference kernel for scaling rocprofv3 byte counters)")
    return p.parse_args()


def streamk_sweep(R=20, rounds=5):
    """The stream-K form of the 256x128 GEMM (fp8q_gemm_blockscaled_streamk,
    one workgroup per CU) against the single-pass kernels: the automatic one
    and the ping-pong kernel (id 5), graph-timed back-to-back launches over
    rotating weight copies (each launch streams its weights from HBM), the
    three variants taking turns `rounds` times (median).  The shapes are the
    ones the automatic stream-K rule was fixed on: a last round of few tiles
    and a long K (M = 1792 and 2560), and shapes where most CUs have a tile
    in the last round (the two prefill projections among them).  Random FP8
    codes (no NaN code), scales uniform in [0, 0.01)."""
    import torch
    import w8a8_fp8_block_amd as fp8q
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    work = torch.empty((fp8q.fp8q_gemm_streamk_workspace_bytes(0),), dtype=torch.uint8, device=dev)

    def codes(shape):
        c = torch.randint(0, 256, shape, generator=gen, dtype=torch.uint8, device=dev)
        c[(c & 0x7F) == 0x7F] = 0
        return c

    for M, N, K in ((1792, 5120, 17408), (2560, 6656, 17408), (2304, 5120, 17408),
                    (2048, 8448, 8192), (3072, 4224, 17408), (4576, 5120, 17408),
                    (1168, 17408, 5120)):
        a = codes((M, K))
        km = torch.rand((K // 128, fp8q.fp8q_m_pad(M)), generator=gen, device=dev) * 0.01
        w_rot = _rotation(codes((N, K)))
        ws = torch.rand((N // 128, K // 128), generator=gen, device=dev) * 0.01
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        fns = {
            "auto": lambda i: fp8q.fp8q_gemm_blockscaled(a, km, w_rot[i % len(w_rot)], ws, out),
            "pingpong": lambda i: fp8q.fp8q_gemm_blockscaled(a, km, w_rot[i % len(w_rot)], ws, out,
                                                             kernel=5),
            "streamk": lambda i: fp8q.fp8q_gemm_blockscaled_streamk(a, km, w_rot[i % len(w_rot)], ws,
                                                                     out, work),
        }
        ts = {k: [] for k in fns}
        for _ in range(rounds):
            for k, fn in fns.items():
                ts[k].append(_b2b_us(fn, R)[0])
        t = {k: round(float(np.median(v)), 2) for k, v in ts.items()}
        tiles = (M + 255) // 256 * (N // 128)
        print(json.dumps({"M": M, "N": N, "K": K, "tiles_256x128": tiles,
                          "auto_kernel": fp8q.fp8q_gemm_select(M, N, K),
                          "streamk_auto": fp8q.fp8q_gemm_streamk_select(M, N, K),
                          "us": t, "streamk_vs_best_single_pass":
                              round(t["streamk"] / min(t["auto"], t["pingpong"]), 3)}), flush=True)
        del a, km, w_rot, ws, out
        torch.cuda.empty_cache()


def quant_vs_copy(reps=20):
    """The quantizer (variant A, row-major scales) beside a plain device copy
    of its bf16 input (torch's copy kernel: 2MK bytes read, 2MK written) at
    the act-quant sweep's M >= 1168 shapes, `reps` launches of each, every one
    after a sum over a 1 GiB buffer (a read, so no write-back of the eviction
    is still draining when the kernel starts).  The durations come from a
    kernel trace of this run; the launches of each shape and kind are
    consecutive, in the order of the JSON lines printed."""
    import torch
    import synth
    import w8a8_fp8_block_amd as fp8q
    dev = torch.device("cuda:0")
    big = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sweep = synth.WORKLOADS["quant_sweep"]
    for K in sorted({w.K for w in sweep}):
        base = next(w for w in sweep if w.K == K)
        for M in sorted({w.M for w in sweep if w.M >= 1168}):
            x = torch.from_numpy(synth.make_inputs(base, M=M, with_weights=False)[0]
                                 .view(np.int16)).to(dev)
            q = torch.empty((M, K), dtype=torch.uint8, device=dev)
            sc = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
            y = torch.empty_like(x)
            for _ in range(reps):
                torch.sum(big)
                fp8q.fp8q_quant_act(x, q, sc, variant=1)
            for _ in range(reps):
                torch.sum(big)
                y.copy_(x)
            torch.cuda.synchronize()
            print(json.dumps({"M": M, "K": K, "quant_bytes": quant_bytes(M, K),
                              "copy_bytes": 4 * M * K, "launches": reps}), flush=True)
            del x, q, sc, y


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
    res["down_kernel"] = fp8q.fp8q_gemm_kernel_name(M, H, I)
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


def gemm_sweep(reps=10, ms=None):
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
        for M in ms or (16, 32, 64, 65, 96, 128, 192, 256, 384, 512, 768, 1024, 1168, 1536, 2048):
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


def gemm_sweep_b2b(R=20, ms=None):
    """The block-scaled GEMM up to 64 rows at three projection shapes, as
    layers run in a model: each variant's R launches back to back (one HIP
    graph, _b2b_us) cycling through copies of the weights that together
    exceed the last-level cache, so every launch streams its weights from
    HBM.  Variants: the automatic single-pass kernel and
    fp8q_gemm_blockscaled_splitk at 2, 3, 4 and 6 splits (and the automatic
    count); the split count fp8q_gemm_splitk_select picks and whether it is
    within 3% of the fastest.  Normal activations, quantized by the library;
    weights normal(0, 0.02), block-quantized."""
    import torch
    import w8a8_fp8_block_amd as fp8q
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    for N, K in ((5120, 17408), (6144, 5120), (17408, 5120)):
        wq, wsc = quantize_weights_gpu(torch.randn((N, K), generator=gen, device=dev) * 0.02)
        w_rot = _rotation(wq)
        for M in ms or (1, 2, 4, 8, 12, 16, 24, 32, 33, 40, 48, 56, 64, 65):
            x = torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16)
            q = torch.empty((M, K), dtype=torch.uint8, device=dev)
            srm = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
            skm = torch.empty((K // 128, fp8q.fp8q_m_pad(M)), dtype=torch.float32, device=dev)
            fp8q.fp8q_quant_act_kmajor(x, q, srm, skm)
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            sel = fp8q.fp8q_gemm_splitk_select(M, N, K)
            t = {"single": _b2b_us(lambda i: fp8q.fp8q_gemm_blockscaled(
                q, skm, w_rot[i % len(w_rot)], wsc, out), R)[0]}
            for S in sorted({2, 3, 4, 6} | ({sel} if sel >= 2 else set())):
                wsp = torch.empty((S * M * N,), dtype=torch.float32, device=dev)
                t[f"s{S}"] = _b2b_us(lambda i: fp8q.fp8q_gemm_blockscaled_splitk(
                    q, skm, w_rot[i % len(w_rot)], wsc, out, wsp, splits=S), R)[0]
                del wsp
            t = {v: round(u, 2) for v, u in t.items()}
            best = min(t, key=t.get)
            chosen = t["single"] if sel < 2 else t[f"s{sel}"]
            print(json.dumps({"M": M, "N": N, "K": K, "auto_kernel": fp8q.fp8q_gemm_select(M, N, K),
                              "us": t, "best": best, "splitk_auto": sel,
                              "rule_ok": chosen <= 1.03 * t[best]}), flush=True)
            del x, q, srm, skm, out
        del w_rot, wq, wsc


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


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        return None


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
    t2 = sum(run(min(2, w.M)))
    R = int(max(2, min(w.M, 2 * budget_s / max(t2, 1e-6))))
    R = max(1, min(R, w.M))
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
    flops = 2.0 * R * w.N * w.K
    return {
        "value": round(flops / t / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {R} of {w.M} rows of {w.desc}: quantize + relayout + fp64 block GEMM "
                  f"({t:.2f} s, one run)",
        "cpu_model": _cpu_model(),
        "quant_relayout_s": round(tq, 4),
        "gemm_s": round(tg, 3),
        "quant_relayout_1thread_s": None if tq1 is None else round(tq1, 4),
    }


def cpu_baseline_quant(w, x_bits, budget_s):
    """Time the oracle's quantizer + relayout on the first R rows (R sized to
    about budget_s), as GB/s of the quantizer's and relayout's algorithmic
    bytes."""
    import oracle
    oracle._load()
    G = w.K // 128

    def run(R):
        xs = np.ascontiguousarray(x_bits[:R])
        t0 = time.perf_counter()
        _, a_s = oracle.quant_act(xs)
        oracle.scale_to_kmajor(a_s)
        return time.perf_counter() - t0
    t1 = run(1)
    R = max(1, min(w.M, int(budget_s / max(t1, 1e-6))))
    t = run(R)
    nbytes = quant_bytes(R, w.K) + 4 * R * G + 4 * m_pad(R) * G
    return {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"first {R} of {w.M} rows of {w.desc}: quantize + relayout ({t:.3f} s, one run)",
            "cpu_model": _cpu_model()}


def m_pad(m):
    return (m + 15) // 16 * 16


def quant_kernel_name(M, K, fused):
    """The quantizer kernel fp8q_proj runs: with both scale layouts the flat
    kernel up to 2^17 scale groups and its tiled form beyond."""
    if not fused:
        return "quant_a_kernel"
    return ("quant_a_tile_kernel" if M * (K // 128) > 1 << 17 else "quant_a_kernel") + \
        " (both scale layouts)"


def quant_bytes(M, K):
    """Algorithmic bytes of the quantizer: 2 read + 1 written per element and
    one fp32 scale per 128-group."""
    return 3 * M * K + 4 * M * (K // 128)


def gemm_stream_bytes(M, N, K):
    """Algorithmic bytes of the GEMM: weights, activation codes, output and
    both scale arrays (the roofline of the weight-streaming decode widths)."""
    G = K // 128
    return N * K + M * K + 2 * M * N + 4 * (N // 128) * G + 4 * m_pad(M) * G


def _rotation(t, target_bytes=600 << 20, cap=64):
    """t and copies of it, at least 2 and at most cap, together at least
    target_bytes where the cap allows: back-to-back launches that cycle
    through them stream from HBM, not from the 256 MB last-level cache."""
    nb = max(1, t.numel() * t.element_size())
    n = int(max(2, min(cap, -(-target_bytes // nb))))
    return [t] + [t.clone() for _ in range(n - 1)]


B2B_METHOD = {"graph": "one HIP graph of R launches (torch.cuda.CUDAGraph), timed replay",
              "stream": "R launches from the host between two events"}


def _b2b_us(fn, R, graph=True):
    """Mean time per launch of R back-to-back launches fn(i): captured into
    one HIP graph and replayed between two HIP events, so that no host launch
    gap sits between the kernels (launches from Python are ~10 us apart,
    longer than the small kernels); plain launches between two events if the
    capture fails.  The timed replay follows B2B_SETTLE_S seconds of the same
    replays.  Returns (us, method)."""
    import torch
    fn(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def settle(run):  # the same launches until the power control has settled
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < B2B_SETTLE_S:
            run()
            torch.cuda.synchronize()
    if graph:
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(R):
                    fn(i)
            settle(g.replay)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / R
            del g
            return us, "graph"
        except Exception as ex:  # capture not possible here: plain launches
            print(f"[bench] graph capture failed ({str(ex).splitlines()[0][:120]}); "
                  "timing plain launches", file=sys.stderr, flush=True)
            torch.cuda.synchronize()

    def launches():
        for i in range(R):
            fn(i)
    settle(launches)
    e0.record()
    launches()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / R, "stream"


# Untimed steps run before the warmup steps, for at least this long: under
# this load the device's power controller overshoots and recovers over the
# first few tens of milliseconds (one trace: the large prefill GEMM at 404 us,
# then 520-530 us, then back to a steady ~400 us within ~25 ms), so a short
# warmup would leave that transient inside the timed steps.
SETTLE_S = 0.3
# the same before each back-to-back measurement (replays of its graph)
B2B_SETTLE_S = 0.15


def _settle(step, seconds):
    """Run step(i) in bursts of 8 (synchronising after each burst) until
    `seconds` of wall time have passed.  Returns (steps run, host time per
    step spent issuing the launches, wall time per step): a step whose issue
    time is most of its wall time is bound by the host's launches, not the
    GPU."""
    import torch
    t0, n, issue = time.perf_counter(), 0, 0.0
    while True:
        t1 = time.perf_counter()
        for _ in range(8):
            step(n)
            n += 1
        issue += time.perf_counter() - t1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n, issue / n, (time.perf_counter() - t0) / n


def _spin_cycles_per_us():
    """Cycles of torch.cuda._sleep per microsecond on this device (its spin
    counts a hardware counter; timed once with events)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    e0.record()
    torch.cuda._sleep(2_000_000)
    e1.record()
    torch.cuda.synchronize()
    return 2_000_000 / (e0.elapsed_time(e1) * 1e3)


class KernelEvents:
    """HIP timing events created with hipEventDisableSystemFence, for the
    per-kernel times inside the timed steps.  A default event (torch's) is a
    system-scope release: recording it writes back and invalidates L2, which
    is charged to the interval it closes and leaves the next kernel a cold L2.
    These events stamp the same points on the stream (each marker waits for
    the work before it) without that fence, so an interval is the kernel's
    own time, as a kernel trace reports it; the region's start and end keep
    torch's fenced events.  Calls torch's HIP runtime (already loaded)."""

    _lib = None

    @classmethod
    def _hip(cls):
        if cls._lib is None:
            import ctypes
            import torch
            lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            for f in ("hipEventCreateWithFlags", "hipEventRecord", "hipEventElapsedTime",
                      "hipEventDestroy"):
                getattr(lib, f).restype = ctypes.c_int
            cls._lib = lib
        return cls._lib

    def __init__(self, n):
        import ctypes
        lib = self._hip()
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = lib.hipEventCreateWithFlags(ctypes.byref(e), 0x20000000)  # hipEventDisableSystemFence
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.ev.append(e)

    def record(self, i, stream):
        rc = self._hip().hipEventRecord(self.ev[i], ctypes_stream(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_us(self, i, j):
        import ctypes
        ms = ctypes.c_float()
        rc = self._hip().hipEventElapsedTime(ctypes.byref(ms), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value * 1e3

    def __del__(self):
        lib = KernelEvents._lib
        if lib is not None:
            for e in getattr(self, "ev", []):
                lib.hipEventDestroy(e)


def ctypes_stream(stream):
    import ctypes
    return ctypes.c_void_p(stream.cuda_stream)


class ClockStamps:
    """Shader clock over a stretch of the stream: a clock stamp before and
    after (fp8q_clock_stamp, 1024 one-wave workgroups over the 8 XCDs),
    paired by CU."""

    def __init__(self, fp8q, dev):
        import torch
        self.fp8q = fp8q
        self.buf = [torch.empty((1024, 4), dtype=torch.int64, device=dev) for _ in range(2)]

    def start(self):
        self.fp8q.fp8q_clock_stamp(self.buf[0])

    def stop(self):
        self.fp8q.fp8q_clock_stamp(self.buf[1])

    def result(self):
        per, pairs = self.fp8q.shader_clock_ghz(self.buf[0].cpu().numpy(), self.buf[1].cpu().numpy())
        if not per:
            return None
        return {"shader_ghz": round(float(np.median(list(per.values()))), 3),
                "per_xcd": {str(k): round(v, 3) for k, v in sorted(per.items())},
                "cu_pairs": pairs,
                "method": "s_memtime / s_memrealtime stamps before and after, paired by CU"}


def _pct(us):
    p10, p50, p90 = np.percentile(np.asarray(us), [10, 50, 90])
    return {"p10_us": round(float(p10), 2), "median_us": round(float(p50), 2),
            "p90_us": round(float(p90), 2)}


def measure_projection(w, steps, warmup, per_row=False, comparators=False, cpu_budget=2.0,
                       R=20):
    """One projection workload on the GPU: the whole step (quantizer, relayout
    or the fused quantizer, GEMM) over `steps` timed steps with HIP events
    around every kernel, the shader clock over those steps, back-to-back
    launches of each kernel, and the oracle on a bounded sample.  Every step
    and every back-to-back launch takes the next of several copies of the
    activations and of the weights (each set at least 600 MB where 64 copies
    reach it), so that its reads come from HBM and not from the 256 MB
    last-level cache.  Returns (entry dict, extras for the benchmark line)."""
    import torch
    import synth
    import w8a8_fp8_block_amd as fp8q
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    M, K, N = w.M, w.K, w.N
    G = K // 128
    print(f"[bench] inputs {w.desc} (seed {w.seed})", file=sys.stderr, flush=True)
    x_bits, wf, _ = synth.make_inputs(w)
    x = torch.from_numpy(x_bits.view(np.int16)).to(dev)
    wq, ws = quantize_weights_gpu(torch.from_numpy(wf).to(dev), per_row)
    # the GEMM with a caller workspace (as fp8q_proj_splitk runs it: stream-K
    # or split-K where the automatic choice takes them); per-row weight
    # scales have the single-pass kernels only
    work = None
    if per_row:
        gemm = fp8q.fp8q_gemm_rowscaled
        gemm_name = fp8q.fp8q_gemm_kernel_name(M, N, K) + " (its per-row weight-scale form)"
    else:
        need = fp8q.fp8q_gemm_splitk_workspace_bytes(M, N, K, 0)
        work = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)

        def gemm(a_, s_, w_, ws_, o_):
            fp8q.fp8q_gemm_blockscaled_splitk(a_, s_, w_, ws_, o_, work)
        if fp8q.fp8q_gemm_streamk_select(M, N, K) == 1:
            gemm_name = fp8q.STREAMK_KERNEL_NAME
        elif fp8q.fp8q_gemm_splitk_select(M, N, K) >= 2:
            gemm_name = "+".join(fp8q.SPLITK_KERNEL_NAMES)
        else:
            gemm_name = fp8q.fp8q_gemm_kernel_name(M, N, K)
    act_q, act_s, act_km = fp8q.alloc_proj_scratch(M, K)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    variant, _, _ = fp8q.fp8q_quant_select(M, K, props.multi_processor_count)
    fused = fp8q.fp8q_proj_quant_fused(M, K)  # the same choice fp8q_proj makes
    clock = ClockStamps(fp8q, dev)
    x_rot, w_rot = _rotation(x), _rotation(wq)

    # timed step j records events 3j+1 (after the quantizer), 3j+2 (after the
    # relayout; not where the quantizer writes the K-major scales itself: an
    # event record right behind another costs ~4 us of device time, and the
    # GEMM interval then opens at 3j+1) and 3j+3 (after the GEMM); event 3j,
    # recorded by the step before (event 0 by the first), opens its quantizer
    # interval
    def step(i, ev=None):
        xi, wi = x_rot[i % len(x_rot)], w_rot[i % len(w_rot)]
        j = i - warmup
        if ev and j == 0: ev.record(0, stream)
        if fused:
            fp8q.fp8q_quant_act_kmajor(xi, act_q, act_s, act_km)
        else:
            fp8q.fp8q_quant_act(xi, act_q, act_s)
        if ev: ev.record(3 * j + 1, stream)
        if not fused:
            fp8q.fp8q_scale_to_kmajor(act_s, act_km)
        if ev and not fused: ev.record(3 * j + 2, stream)
        gemm(act_q, act_km, wi, ws, out)
        if ev: ev.record(3 * j + 3, stream)

    settle_steps, issue_s, settle_step_s = _settle(step, SETTLE_S)
    # Where issuing a step's launches from Python takes most of its wall time
    # (the small workloads), the GPU would idle between kernels, inside the
    # event intervals; there the timed steps are all issued behind a GPU spin
    # (torch.cuda._sleep) long enough to cover their issue, so that they run
    # back to back as a graph or a native caller would run them, and the wall
    # time starts once the GPU has reached the first of them.
    host_bound = issue_s > 0.5 * settle_step_s
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = KernelEvents(3 * steps + 1)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    spin_us = 1.5 * issue_s * 1e6 * steps + 2000.0 if host_bound else 0.0
    if spin_us:
        cyc = _spin_cycles_per_us()
    print(f"[bench] timing {steps} steps of {w.desc}" +
          (f" (issued behind a {spin_us / 1e3:.1f} ms spin)" if spin_us else ""),
          file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    if spin_us:
        torch.cuda._sleep(int(spin_us * cyc))
    clock.start()
    t_start.record(stream)
    for i in range(steps):
        step(warmup + i, evs)
    t_end.record(stream)
    clock.stop()
    if spin_us:
        t_start.synchronize()
        wall0 = time.perf_counter()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = t_start.elapsed_time(t_end)
    # The step time is the timed steps' span between the two events on the
    # stream.  The host's wall time over the same stretch (kept in the line)
    # starts on an idle device and adds ~0.65 ms before the first kernel
    # runs, which no step of a running job pays; where the steps were issued
    # behind the spin it starts once the device reached them, and the larger
    # of the two is taken.
    ms_per_step = (max(gpu_ms, wall * 1e3) if spin_us else gpu_ms) / steps
    quant_us = np.array([evs.elapsed_us(3 * i, 3 * i + 1) for i in range(steps)])
    g0 = 1 if fused else 2
    relay_us = None if fused else np.array([evs.elapsed_us(3 * i + 1, 3 * i + 2) for i in range(steps)])
    gemm_us = np.array([evs.elapsed_us(3 * i + g0, 3 * i + 3) for i in range(steps)])
    step_clock = clock.result()
    # the same step captured R times into one HIP graph (no host launch gaps)
    step_graph_us, step_graph_how = _b2b_us(lambda i: step(i), R)

    # back-to-back launches of each kernel, cycling through the input copies
    gclock = ClockStamps(fp8q, dev)
    gclock.start()
    gemm_b2b, b2b_how = _b2b_us(lambda i: gemm(act_q, act_km, w_rot[i % len(w_rot)], ws, out), R)
    gclock.stop()
    torch.cuda.synchronize()
    gemm_b2b_clock = gclock.result()
    if fused:
        quant_b2b, _ = _b2b_us(lambda i: fp8q.fp8q_quant_act_kmajor(x_rot[i % len(x_rot)], act_q,
                                                                   act_s, act_km), R)
        relay_b2b = None
    else:
        quant_b2b, _ = _b2b_us(lambda i: fp8q.fp8q_quant_act(x_rot[i % len(x_rot)], act_q, act_s), R)
        relay_b2b, _ = _b2b_us(lambda i: fp8q.fp8q_scale_to_kmajor(act_s, act_km), R)
    del x_rot, w_rot

    flops = 2.0 * M * N * K
    kern = fp8q.fp8q_gemm_select(M, N, K)
    gemm_avg = float(np.mean(gemm_us))
    if kern == 2:
        # decode and small widths: the GEMM streams the weight matrix (HBM-bound)
        gbytes = gemm_stream_bytes(M, N, K)
        roofline = {"bound": "hbm", "kernel": gemm_name,
                    "achieved": round(gbytes / gemm_avg / 1e3, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(gbytes / gemm_avg / 1e3 / HBM_PEAK_GBS, 4),
                    "traffic": None, "avg_launch_us": round(gemm_avg, 2), **_pct(gemm_us),
                    "back_to_back_us": round(gemm_b2b, 2),
                    "back_to_back_achieved": round(gbytes / gemm_b2b / 1e3, 1),
                    "back_to_back_frac": round(gbytes / gemm_b2b / 1e3 / HBM_PEAK_GBS, 4),
                    "algorithmic_bytes_per_launch": gbytes}
    else:
        roofline = {"bound": "mfma", "kernel": gemm_name,
                    "achieved": round(flops / gemm_avg / 1e6, 2), "peak": FP8_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(flops / gemm_avg / 1e6 / FP8_PEAK_TFLOPS, 4),
                    "traffic": (gemm_traffic() if w.name == "large_prefill" and not per_row
                                else None),
                    "avg_launch_us": round(gemm_avg, 2), **_pct(gemm_us),
                    "back_to_back_us": round(gemm_b2b, 2),
                    "back_to_back_achieved": round(flops / gemm_b2b / 1e6, 2),
                    "back_to_back_frac": round(flops / gemm_b2b / 1e6 / FP8_PEAK_TFLOPS, 4),
                    "algorithmic_flops_per_launch": flops}
    roofline["back_to_back_method"] = B2B_METHOD[b2b_how]
    if gemm_b2b_clock:
        roofline["back_to_back_shader_ghz"] = gemm_b2b_clock["shader_ghz"]
    qb = quant_bytes(M, K) + (4 * m_pad(M) * G if fused else 0)
    qavg = float(np.mean(quant_us))
    act_quant = {"kernel": quant_kernel_name(M, K, fused),
                 "achieved": round(qb / qavg / 1e3, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(qb / qavg / 1e3 / HBM_PEAK_GBS, 4),
                 "avg_launch_us": round(qavg, 2), **_pct(quant_us),
                 "back_to_back_us": round(quant_b2b, 2),
                 "back_to_back_achieved": round(qb / quant_b2b / 1e3, 1),
                 "back_to_back_frac": round(qb / quant_b2b / 1e3 / HBM_PEAK_GBS, 4),
                 "algorithmic_bytes_per_launch": qb}
    entry = {
        "workload": f"{w.name} M={M} K={K} N={N}",
        "ms_per_step": round(ms_per_step, 5),
        "tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "step_graph_us": round(step_graph_us, 2),
        "step_graph_tflops": round(flops / step_graph_us / 1e6, 2),
        "step_graph_method": B2B_METHOD[step_graph_how],
        "step": ("act-quant writing both scale layouts" if fused else
                 "act-quant + scale relayout") +
                (" + per-row-scaled FP8 GEMM" if per_row else
                 " + block-scaled FP8 GEMM (workspace form, automatic choice)"),
        "quant_variant": "B" if variant == 2 else "A",
        "roofline": roofline,
        "act_quant": act_quant,
        "clock": step_clock,
        "settle": {"seconds": SETTLE_S, "steps": settle_steps},
        "timed_region": {"gpu_event_ms": round(gpu_ms, 4), "wall_ms": round(wall * 1e3, 4)},
        "issue": {"host_us_per_step": round(issue_s * 1e6, 1),
                  "settle_wall_us_per_step": round(settle_step_s * 1e6, 1),
                  "timed_steps_issued_behind_spin_ms": round(spin_us / 1e3, 2)},
    }
    if not fused:
        rb = 4 * M * G + 4 * m_pad(M) * G
        entry["relayout"] = {"kernel": "relayout_kernel", "avg_launch_us": round(float(np.mean(relay_us)), 2),
                             "back_to_back_us": round(relay_b2b, 2),
                             "back_to_back_GBs": round(rb / relay_b2b / 1e3, 1),
                             "algorithmic_bytes_per_launch": rb}

    extras = {}
    if comparators:
        extras = _comparators(fp8q, dev, stream, x, act_q, wq, ws, per_row, M, N, K, gemm_b2b, R)
    del x, wq, ws, act_q, act_s, act_km, out, work
    torch.cuda.empty_cache()
    if cpu_budget:
        print(f"[bench] cpu baseline (oracle) {w.desc}", file=sys.stderr, flush=True)
        entry["cpu_baseline"] = cpu_baseline(w, x_bits, wf, cpu_budget, per_row)
    return entry, extras


def _comparators(fp8q, dev, stream, x, act_q, wq, ws, per_row, M, N, K, gemm_b2b_us, R):
    """bf16 comparator (our bf16 MFMA kernel and hipBLASLt) on the weights
    dequantized once by fp8q_dequant_fp8_bf16, and, for context, hipBLASLt's
    FP8 GEMM with per-tensor / per-row scales; back-to-back launches."""
    import torch
    flops = 2.0 * M * N * K
    wd = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    fp8q.fp8q_dequant_fp8_bf16(wq, ws, wd, per_row)
    xb = x.view(torch.bfloat16)
    outb = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    wds = [wd, wd.clone()]
    bf16_own_us, _ = _b2b_us(lambda i: fp8q.fp8q_gemm_bf16(xb, wds[i % 2], outb), R)
    wts = [t.t().contiguous() for t in wds]  # [K,N] for a plain (non-batched) mm
    del wds
    bf16_lib_us, _ = _b2b_us(lambda i: torch.mm(xb, wts[i % 2], out=outb), R, graph=False)
    del wts, wd
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
                us, _ = _b2b_us(lambda i: torch._scaled_mm(a8, w8s[i % 2].t(), scale_a=sa, scale_b=sb,
                                                           out_dtype=torch.bfloat16), R, graph=False)
                fp8_lib[name] = {"us": round(us, 2), "tflops": round(flops / us / 1e6, 1)}
            except Exception as ex:  # not offered on this build / device
                fp8_lib[name] = {"error": str(ex).splitlines()[0][:160]}
        del w8s
    del outb
    return {
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


def measure_quant_shape(w, R=20, cpu_budget=0.3):
    """The act-quant + scale-relayout step on one quantizer-sweep shape, as
    fp8q_proj runs it (one kernel writing both scale layouts up to 2^19 scale
    groups, else the quantizer and the relayout; with the row-major-only
    quantizer timed beside the one kernel, for reference): back-to-back launches over
    rotating input copies (at least 600 MB where 64 copies reach it), the
    quantizer's GB/s against the HBM peak, and the oracle on a bounded
    sample."""
    import torch
    import synth
    import w8a8_fp8_block_amd as fp8q
    dev = torch.device("cuda:0")
    M, K = w.M, w.K
    G = K // 128
    x_bits, _, _ = synth.make_inputs(w, with_weights=False)
    x = torch.from_numpy(x_bits.view(np.int16)).to(dev)
    q, s, km = fp8q.alloc_proj_scratch(M, K)
    fused = fp8q.fp8q_proj_quant_fused(M, K)
    x_rot = _rotation(x)
    if fused:
        tq, how = _b2b_us(lambda i: fp8q.fp8q_quant_act_kmajor(x_rot[i % len(x_rot)], q, s, km), R)
        tr = 0.0
        t_rm, _ = _b2b_us(lambda i: fp8q.fp8q_quant_act(x_rot[i % len(x_rot)], q, s), R)
    else:
        tq, how = _b2b_us(lambda i: fp8q.fp8q_quant_act(x_rot[i % len(x_rot)], q, s), R)
        tr, _ = _b2b_us(lambda i: fp8q.fp8q_scale_to_kmajor(s, km), R)
    del x_rot, x, q, s, km
    qb = quant_bytes(M, K) + (4 * m_pad(M) * G if fused else 0)
    rb = 4 * M * G + 4 * m_pad(M) * G
    e = {"M": M, "K": K, "path": "fused (both scale layouts)" if fused else "quantizer + relayout",
         "roofline": {"bound": "hbm", "kernel": quant_kernel_name(M, K, fused),
                      "achieved": round(qb / tq / 1e3, 1),
                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(qb / tq / 1e3 / HBM_PEAK_GBS, 4), "traffic": None,
                      "back_to_back_us": round(tq, 2), "back_to_back_method": B2B_METHOD[how],
                      "algorithmic_bytes_per_launch": qb},
         "step_us": round(tq + tr, 2),
         "step_GBs": round((qb + (rb if not fused else 0)) / (tq + tr) / 1e3, 1)}
    if not fused:
        e["relayout_back_to_back_us"] = round(tr, 2)
    else:
        # the row-major-only quantizer (fp8q_quant_act, no K-major output) on
        # the same input: what the step would pay before a separate relayout
        qrm = quant_bytes(M, K)
        e["rowmajor_quantizer"] = {"kernel": "quant_a_kernel (row-major scales only)",
                                   "back_to_back_us": round(t_rm, 2),
                                   "frac": round(qrm / t_rm / 1e3 / HBM_PEAK_GBS, 4)}
    if cpu_budget:
        e["cpu_baseline"] = cpu_baseline_quant(w, x_bits, cpu_budget)
    return e


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
    if args.quant_vs_copy:
        quant_vs_copy()
        return
    if args.streamk_sweep:
        streamk_sweep()
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
        gemm_sweep(ms=[int(v) for v in args.sweep_m.split(",")] if args.sweep_m else None)
        return
    if args.gemm_sweep_b2b:
        gemm_sweep_b2b(ms=[int(v) for v in args.sweep_m.split(",")] if args.sweep_m else None)
        return

    import torch
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    w = (synth.workload(args.workload, M=args.M) if args.workload == "decode"
         else synth.workload(args.workload))
    per_row = args.weights == "row"
    budget = 0 if args.no_cpu_baseline else args.cpu_seconds
    main_entry, extras = measure_projection(w, args.steps, args.warmup, per_row=per_row,
                                            comparators=True, cpu_budget=budget)

    # the other configurations, each with its own roofline and oracle baseline
    configs = {}
    if not args.only_workload:
        small = 0 if args.no_cpu_baseline else 2.0
        for name in ("tiny", "decode", "prefill", "large_prefill"):
            for cw in synth.WORKLOADS[name]:
                if cw == w:
                    continue
                key = name if len(synth.WORKLOADS[name]) == 1 else f"{name}_M{cw.M}"
                configs[key], _ = measure_projection(cw, args.steps, args.warmup, per_row=per_row,
                                                     cpu_budget=small)
        print("[bench] quantizer sweep", file=sys.stderr, flush=True)
        configs["quant_sweep"] = [
            measure_quant_shape(qw, cpu_budget=0 if args.no_cpu_baseline else 0.3)
            for qw in synth.WORKLOADS["quant_sweep"]]

    M, K, N = w.M, w.K, w.N
    flops = 2.0 * M * N * K
    rec = {
        "metric": "block-scaled FP8 proj TFLOP/s (M=4576) + act-quant GB/s vs HBM peak",
        "value": main_entry["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_entry["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": main_entry["workload"],
            "M": M, "K": K, "N": N,
            "activations": f"bf16 {w.dist}(0,1), {w.n_outliers} outlier channels x{w.outlier_factor:g}",
            "weights": ("fp8 e4m3 [N,K], fp32 scale per row (from N(0,0.02))" if per_row else
                        "fp8 e4m3 [N,K], fp32 scale per 128x128 block (from N(0,0.02))"),
            "output": "bf16 [M,N]",
            "step": main_entry["step"],
            "quant_variant": main_entry["quant_variant"],
            "device": props.name, "gcn_arch": props.gcnArchName,
            "cus": props.multi_processor_count,
        },
        "roofline": main_entry["roofline"],
        "act_quant": main_entry["act_quant"],
        "cpu_baseline": main_entry.get("cpu_baseline"),
        "clock": main_entry["clock"],
        "settle": main_entry["settle"],
        "timed_region": main_entry["timed_region"],
        "step_graph_us": main_entry["step_graph_us"],
        "step_graph_tflops": main_entry["step_graph_tflops"],
        "step_graph_method": main_entry["step_graph_method"],
    }
    if "relayout" in main_entry:
        rec["relayout"] = main_entry["relayout"]
    rec.update(extras)
    rec["configs"] = configs
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
