"""GPU parity of the split-K form of the block-scaled FP8 GEMM
(fp8q_gemm_blockscaled_splitk) against the oracle's fp64 block-form product,
with the same accuracy contract as the single-pass kernels (rel_rms <= 1e-3
against the bf16-rounded reference; per element |o - r| <= ulp_bf16(r) +
1e-3*RMS(r)).  Split counts that do and do not divide the K-block count,
one block per split, ragged row tiles, exact special cases that must match
bit for bit, workspace and output canaries, and run-to-run reproducibility.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import Guarded, bf16_bits_to_f64, dev, host, log, require_gpu

pytestmark = pytest.mark.gpu

fp8q = None
RTOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global fp8q
    require_gpu()
    import w8a8_fp8_block_amd as m
    fp8q = m
    yield


def _splitk_gpu(orc, a, a_s, wq, ws, splits, km=None):
    M, K = a.shape
    N = wq.shape[0]
    if km is None:
        km = orc.scale_to_kmajor(a_s)
    need = fp8q.fp8q_gemm_splitk_workspace_bytes(M, N, K, splits)
    out = Guarded((M, N), torch.int16)
    work = Guarded((max(need, 16) // 4,), torch.float32, fill=0x7F) if need else None
    fp8q.fp8q_gemm_blockscaled_splitk(dev(a), dev(km), dev(wq), dev(ws), out.t,
                                      None if work is None else work.t, splits=splits)
    torch.cuda.synchronize()
    out.check_canary()
    if work is not None:
        work.check_canary()
    return bf16_bits_to_f64(host(out.t))


def _assert_tol(o, r, what, rms=None):
    import oracle
    rel, exc, relf = oracle.gemm_errors(o, r, rms)
    log(f"  {what}: rel_rms={rel:.3e} (vs fp64 {relf:.3e}) worst/bound={exc:.3f}")
    assert rel <= RTOL, f"{what}: rel_rms {rel}"
    assert exc <= 1.0, f"{what}: per-element error {exc} x bound"


def _random_operands(orc, M, N, K, seed, dist="normal"):
    rng = np.random.default_rng(seed)
    v = rng.laplace(0, 1, (M, K)) if dist == "laplace" else rng.standard_normal((M, K))
    x = synth.f32_to_bf16_bits(v.astype(np.float32))
    a, a_s = orc.quant_act(x)
    wq, ws = orc.quant_weight_block(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    return a, a_s, wq, ws


# (M, N, K, splits): K blocks 7 over 2/3/7 splits (uneven ranges and one block
# each), ragged row tiles (130, 257, 300), one row, several column tiles.
@pytest.mark.parametrize("M,N,K,splits", [(130, 384, 896, 2), (130, 384, 896, 3),
                                          (130, 384, 896, 7), (1, 128, 256, 2),
                                          (257, 256, 1280, 4), (300, 512, 2048, 5),
                                          (64, 256, 640, 5), (17, 128, 4096, 8)])
def test_splitk_full(orc, M, N, K, splits):
    a, a_s, wq, ws = _random_operands(orc, M, N, K, M * 31 + N + K + splits)
    ref = orc.gemm_ref(a, a_s, wq, ws)
    log(f"splitk M={M} N={N} K={K} splits={splits}")
    _assert_tol(_splitk_gpu(orc, a, a_s, wq, ws, splits), ref, f"M{M}N{N}K{K}s{splits}")


def test_splitk_auto_falls_back_without_workspace(orc):
    """splits = 0 where the selector gives 1: the single-pass automatic kernel
    runs, no workspace is needed, and the output equals fp8q_gemm_blockscaled's
    bit for bit."""
    M, N, K = 40, 256, 512
    assert fp8q.fp8q_gemm_splitk_select(M, N, K) == 1
    assert fp8q.fp8q_gemm_splitk_workspace_bytes(M, N, K, 0) == 0
    a, a_s, wq, ws = _random_operands(orc, M, N, K, 3)
    o = _splitk_gpu(orc, a, a_s, wq, ws, 0)
    km = orc.scale_to_kmajor(a_s)
    out = torch.empty((M, N), dtype=torch.int16, device="cuda")
    fp8q.fp8q_gemm_blockscaled(dev(a), dev(km), dev(wq), dev(ws), out)
    torch.cuda.synchronize()
    assert np.array_equal(o, bf16_bits_to_f64(host(out)))


def test_splitk_small_integers_exact(orc):
    """Small-integer codes and power-of-two scales: every partial sum and the
    sum of the splits' partials are exact in fp32, so the output is the bf16
    rounding of the exact value, whatever the split."""
    M, N, K = 37, 256, 1536
    G = K // 128
    rng = np.random.default_rng(4)
    a = orc.e4m3_encode(rng.integers(-3, 4, (M, K)).astype(np.float32))
    wq = orc.e4m3_encode(rng.integers(-3, 4, (N, K)).astype(np.float32))
    a_s = np.exp2(rng.integers(-2, 3, (M, G))).astype(np.float32)
    ws = np.exp2(rng.integers(-2, 3, (N // 128, G))).astype(np.float32)
    ref = orc.gemm_ref(a, a_s, wq, ws)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    want = bf16_bits_to_f64(synth.f32_to_bf16_bits(ref.astype(np.float32)))
    for splits in (2, 3, 5, 12):
        assert np.array_equal(_splitk_gpu(orc, a, a_s, wq, ws, splits), want), splits


def test_splitk_block_scale_isolation_exact(orc):
    """All codes 1.0, a_s[m,g] = 2^(m%5), w_s[nb,g] = 2^g * (nb+1): a K block
    read with another block's scale, or a split's range taken twice or not at
    all, changes the exact fp32 result and so its bf16 rounding."""
    M, N, K = 40, 384, 1024
    G = K // 128
    a = np.full((M, K), 0x38, dtype=np.uint8)
    wq = np.full((N, K), 0x38, dtype=np.uint8)
    a_s = np.array([[2.0 ** (m % 5)] * G for m in range(M)], dtype=np.float32)
    ws = np.array([[2.0 ** g * (nb + 1) for g in range(G)] for nb in range(N // 128)],
                  dtype=np.float32)
    ref = orc.gemm_ref(a, a_s, wq, ws)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)  # exact in fp32
    want = bf16_bits_to_f64(synth.f32_to_bf16_bits(ref.astype(np.float32)))
    for splits in (2, 3, 8):
        assert np.array_equal(_splitk_gpu(orc, a, a_s, wq, ws, splits), want), splits


def test_splitk_repeatable(orc):
    """Same inputs, same bits, run to run (the reduction order is fixed)."""
    a, a_s, wq, ws = _random_operands(orc, 200, 256, 2048, 9, "laplace")
    for splits in (3, 6):
        o1 = _splitk_gpu(orc, a, a_s, wq, ws, splits)
        o2 = _splitk_gpu(orc, a, a_s, wq, ws, splits)
        assert np.array_equal(o1, o2)


def _sample_idx(M, N, per_tile, seed=0):
    rng = np.random.default_rng(seed)
    ms, ns = [], []
    for m0 in range(0, M, 128):
        for n0 in range(0, N, 128):
            ms.append(rng.integers(m0, min(m0 + 128, M), per_tile))
            ns.append(rng.integers(n0, n0 + 128, per_tile))
    ms.append(np.full(N // 128, M - 1))
    ns.append(np.arange(0, N, 128) + 127)
    return np.concatenate(ms), np.concatenate(ns)


@pytest.mark.parametrize("M,N,K", [(512, 5120, 17408), (200, 6144, 5120)])
def test_splitk_projection_shapes_sampled(orc, M, N, K):
    """Medium row counts at the down- and a gate/up-projection shape, with the
    automatic split count and one more: outputs sampled in every tile (the
    ragged last row tile included) against the oracle."""
    a, a_s, wq, ws = _random_operands(orc, M, N, K, M + K, "laplace")
    ms, ns = _sample_idx(M, N, per_tile=6)
    log(f"oracle M={M} N={N} K={K} samples={len(ms)}")
    ref = orc.gemm_ref_at(a, a_s, wq, ws, ms, ns)
    rms = float(np.sqrt(np.mean(ref * ref)))
    auto = fp8q.fp8q_gemm_splitk_select(M, N, K)
    for splits in sorted({0, 2, max(auto, 2) + 1}):
        log(f"splitk M={M} N={N} K={K} splits={splits} (auto {auto})")
        o = _splitk_gpu(orc, a, a_s, wq, ws, splits)
        assert np.all(np.isfinite(o))
        _assert_tol(o[ms, ns], ref, f"M{M}N{N}K{K}s{splits}", rms)


@pytest.mark.parametrize("M,N,K", [(200, 1024, 5120), (96, 6144, 5120), (40, 512, 2048)])
def test_proj_splitk(orc, M, N, K):
    """fp8q_proj_splitk: the quantizer's codes and both scale layouts as
    fp8q_proj writes them (bit-exact against the oracle), the output equal bit
    for bit to fp8q_gemm_blockscaled_splitk (splits = 0) on those codes, and
    within the projection tolerance of the oracle; where the selector does not
    split (M = 40) the workspace may be absent and the output is fp8q_proj's."""
    rng = np.random.default_rng(M + N)
    x = synth.f32_to_bf16_bits((rng.standard_normal((M, K)) *
                                np.exp(rng.uniform(-2, 2, (M, 1)))).astype(np.float32))
    wq, ws = orc.quant_weight_block(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    a, a_s = orc.quant_act(x)
    splits = fp8q.fp8q_gemm_splitk_select(M, N, K)
    need = fp8q.fp8q_gemm_splitk_workspace_bytes(M, N, K, 0)
    log(f"proj_splitk M={M} N={N} K={K} splits={splits}")
    out = Guarded((M, N), torch.int16)
    aq = Guarded((M, K), torch.uint8)
    asr = Guarded((M, K // 128), torch.float32)
    askm = Guarded((K // 128, synth.ceil16(M)), torch.float32, fill=0x7F)
    work = Guarded((need // 4,), torch.float32, fill=0x7F) if need else None
    fp8q.fp8q_proj_splitk(dev(x), dev(wq), dev(ws), out.t, aq.t, asr.t, askm.t,
                          None if work is None else work.t)
    torch.cuda.synchronize()
    for gd in (out, aq, asr, askm) + ((work,) if work is not None else ()):
        gd.check_canary()
    assert np.array_equal(host(aq.t), a)
    assert np.array_equal(host(asr.t).view(np.uint32), a_s.view(np.uint32))
    assert np.array_equal(host(askm.t).view(np.uint32), orc.scale_to_kmajor(a_s).view(np.uint32))
    o = bf16_bits_to_f64(host(out.t))
    if splits >= 2:
        assert np.array_equal(o, _splitk_gpu(orc, a, a_s, wq, ws, 0))
    else:
        assert need == 0
        ref_out = torch.empty((M, N), dtype=torch.int16, device="cuda")
        fp8q.fp8q_proj(dev(x), dev(wq), dev(ws), ref_out, aq.t, asr.t, askm.t)
        torch.cuda.synchronize()
        assert np.array_equal(o, bf16_bits_to_f64(host(ref_out)))
    _assert_tol(o, orc.gemm_ref(a, a_s, wq, ws), f"proj_splitk M{M}N{N}K{K}")
