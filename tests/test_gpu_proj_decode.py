"""GPU parity of the whole projection (fp8q_proj) at decode widths, M <= 16,
where its GEMM is the decode kernel.

Against the oracle: the codes and both scale layouts written to the scratch
arrays match the oracle's quantizer bit for bit (K-major pad slots +0), and
the output is within the GEMM tolerance of the oracle's fp64 product.  The
output is also bit-identical to fp8q_gemm_blockscaled with the decode kernel
forced (kernel 2) on the oracle's codes and scales.  Shapes cover one to
sixteen rows, ragged column ranges (N = 5248), short last 1 KB pieces
(K = 2176, 1152, 384), six K slots a wave (K = 6144), grids of fewer
workgroups than CUs (N = 256, 384); groups of zeros, groups whose scale is
below 2^-100 (the quantizer's divide path), signed zeros and magnitudes
around 1e36.  Also: fp8q_proj_splitk gives the same bits, and a captured
graph of the call replays to the eager result.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import Guarded, assert_tol, bf16_bits_to_f64, dev, host, log, require_gpu

pytestmark = pytest.mark.gpu

fp8q = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global fp8q
    require_gpu()
    import w8a8_fp8_block_amd as m
    fp8q = m
    yield


CASES = [(16, 6144, 5120), (1, 6144, 5120), (3, 5248, 2176), (7, 4096, 1152),
         (15, 6144, 6144), (16, 256, 512), (9, 384, 384), (12, 5248, 5120)]


def _inputs(M, N, K, seed):
    """Laplace(0,1) activations with a few outlier channels, and the special
    groups named in the module docstring; normal(0, 0.02) weights."""
    rng = np.random.default_rng(seed)
    x = rng.laplace(0.0, 1.0, (M, K)).astype(np.float32)
    x[:, rng.choice(K, size=max(1, K // 200), replace=False)] *= 50.0
    G = K // 128
    x[0, 128 * (1 % G):128 * (1 % G) + 128] = 0.0                       # all-zero group
    b = 2 % G
    x[M - 1, 128 * b:128 * b + 128] *= 1e-33                            # scale < 2^-100
    b = (G - 1)
    x[M // 2, 128 * b:128 * b + 128] = rng.uniform(-1.0e36, 1.0e36, 128)  # huge magnitudes
    x[M // 2, 128 * b] = -0.0
    x[0, 5] = -0.0
    wf = rng.normal(0.0, 0.02, (N, K)).astype(np.float32)
    return synth.f32_to_bf16_bits(x), wf


def _proj(x, wq, ws, M, N, K, splitk=False):
    out = Guarded((M, N), torch.int16)
    aq = Guarded((M, K), torch.uint8)
    asr = Guarded((M, K // 128), torch.float32)
    askm = Guarded((K // 128, synth.ceil16(M)), torch.float32, fill=0x7F)
    if splitk:
        need = fp8q.fp8q_gemm_splitk_workspace_bytes(M, N, K, 0)
        work = torch.empty((max(need, 16),), dtype=torch.uint8, device="cuda")
        fp8q.fp8q_proj_splitk(x, wq, ws, out.t, aq.t, asr.t, askm.t, work)
    else:
        fp8q.fp8q_proj(x, wq, ws, out.t, aq.t, asr.t, askm.t)
    torch.cuda.synchronize()
    for g in (out, aq, asr, askm):
        g.check_canary()
    return host(out.t), host(aq.t), host(asr.t), host(askm.t)


@pytest.mark.parametrize("M,N,K", CASES)
def test_proj_decode(orc, M, N, K):
    assert fp8q.fp8q_gemm_kernel_name(M, N, K).startswith("gemm_decode_kernel<")
    x, wf = _inputs(M, N, K, seed=M * 7919 + N + K)
    a, a_s = orc.quant_act(x)
    km = orc.scale_to_kmajor(a_s)
    wq, ws = orc.quant_weight_block(wf)
    log(f"decode projection M={M} N={N} K={K} ({fp8q.fp8q_gemm_kernel_name(M, N, K)})")
    xd, wqd, wsd = dev(x), dev(wq), dev(ws)
    out, aq, asr, askm = _proj(xd, wqd, wsd, M, N, K)
    assert np.array_equal(aq, a), "codes"
    assert np.array_equal(asr.view(np.uint32), a_s.view(np.uint32)), "row-major scales"
    assert np.array_equal(askm.view(np.uint32), km.view(np.uint32)), "K-major scales"
    # the GEMM alone on the oracle's codes: the same bits
    o2 = Guarded((M, N), torch.int16)
    fp8q.fp8q_gemm_blockscaled(dev(a), dev(km), wqd, wsd, o2.t, kernel=2)
    torch.cuda.synchronize()
    o2.check_canary()
    assert np.array_equal(out, host(o2.t)), "not the decode kernel's output"
    assert_tol(bf16_bits_to_f64(out), orc.gemm_ref(a, a_s, wq, ws), f"proj M={M} N={N} K={K}")
    again = _proj(xd, wqd, wsd, M, N, K)
    for u, v in zip(again, (out, aq, asr, askm)):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), "not repeatable"


def test_proj_splitk_decode(orc):
    """fp8q_proj_splitk at a decode width (no split there) writes the same
    bits as fp8q_proj."""
    M, N, K = 16, 6144, 5120
    x, wf = _inputs(M, N, K, seed=5)
    wq, ws = orc.quant_weight_block(wf)
    xd, wqd, wsd = dev(x), dev(wq), dev(ws)
    r1 = _proj(xd, wqd, wsd, M, N, K)
    r2 = _proj(xd, wqd, wsd, M, N, K, splitk=True)
    for u, v in zip(r1, r2):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_proj_decode_graph_replay(orc):
    """Captured into a HIP graph and replayed several times, with eager work
    between the replays: every replay gives the eager result."""
    M, N, K = 16, 6144, 5120
    x, wf = _inputs(M, N, K, seed=11)
    wq, ws = orc.quant_weight_block(wf)
    xd, wqd, wsd = dev(x), dev(wq), dev(ws)
    ref = _proj(xd, wqd, wsd, M, N, K)
    out = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    aq = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    asr = torch.zeros((M, K // 128), dtype=torch.float32, device="cuda")
    askm = torch.zeros((K // 128, synth.ceil16(M)), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fp8q.fp8q_proj(xd, wqd, wsd, out, aq, asr, askm)  # warm up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8q.fp8q_proj(xd, wqd, wsd, out, aq, asr, askm)
    for rep in range(3):
        for t in (out, aq, asr, askm):
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (host(out), host(aq), host(asr), host(askm))
        for u, v in zip(got, ref):
            assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), f"replay {rep}"
