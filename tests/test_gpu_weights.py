"""GPU parity of the per-row FP8 weight format and the FP8 -> bf16 weight
dequantizer (page "dispatch_proj.rs", dequant_fp8_bf16_into: one scale index
formula for 128x128 block scales and per-row scales).

* fp8q_dequant_fp8_bf16 bit-exact against the oracle, both geometries,
  ragged N, K not a multiple of 128 for per-row scales, full prefill size;
* fp8q_gemm_rowscaled within the GEMM tolerance of the oracle's fp64 product
  for every kernel the API can force up to decode sizes, and all outputs of
  the automatic, 128x128 and ping-pong kernels at the large prefill size; the
  tiled kernels bit-identical to each
  other; exact special cases bit-exact;
* fp8q_proj_rowscaled end to end on both quantizer paths.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import Guarded, bf16_bits_to_f64, dev, host, log, require_gpu, assert_tol

pytestmark = pytest.mark.gpu

fp8q = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global fp8q
    require_gpu()
    import w8a8_fp8_block_amd as m
    fp8q = m
    yield


def _codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x00  # no NaN codes
    return c


def _dequant_gpu(codes, scale, per_row):
    N, K = codes.shape
    out = Guarded((N, K), torch.int16)
    fp8q.fp8q_dequant_fp8_bf16(dev(codes), dev(scale), out.t, per_row)
    torch.cuda.synchronize()
    out.check_canary()
    return host(out.t).view(np.uint16)


@pytest.mark.parametrize("N,K", [(1, 128), (300, 384), (128, 1280), (1000, 2048)])
def test_dequant_bit_exact(orc, N, K):
    rng = np.random.default_rng(N + K)
    codes = _codes(rng, (N, K))
    s_row = (rng.random(N) * 0.01 + 1e-6).astype(np.float32)
    s_blk = (rng.random(((N + 127) // 128, K // 128)) * 0.01 + 1e-6).astype(np.float32)
    log(f"dequant N={N} K={K}")
    assert np.array_equal(_dequant_gpu(codes, s_row, True), orc.dequant_fp8_bf16(codes, s_row))
    assert np.array_equal(_dequant_gpu(codes, s_blk, False), orc.dequant_fp8_bf16(codes, s_blk))


def test_dequant_rows_k_not_multiple_of_128(orc):
    rng = np.random.default_rng(3)
    codes = _codes(rng, (37, 80))
    s_row = np.ldexp(1.0, rng.integers(-12, 4, 37)).astype(np.float32)
    got = _dequant_gpu(codes, s_row, True)
    assert np.array_equal(got, orc.dequant_fp8_bf16(codes, s_row))


def test_dequant_prefill_weights(orc):
    """The prefill workload's weights (N=17408, K=5120), both formats."""
    w = synth.workload("prefill")
    _, wf, _ = synth.make_inputs(w, M=1)
    for quant in (orc.quant_weight_block, orc.quant_weight_row):
        q, s = quant(wf)
        log(f"dequant prefill weights {quant.__name__}")
        assert np.array_equal(_dequant_gpu(q, s, s.ndim == 1), orc.dequant_fp8_bf16(q, s))


# ---------------------------------------------------------------- GEMM
def _kernels_for(M):
    return (0, 1, 2, 3, 4, 5)


def _gemm_row_gpu(orc, a, a_s, wq, s_row, kernel=0):
    M, K = a.shape
    N = wq.shape[0]
    km = orc.scale_to_kmajor(a_s)
    out = Guarded((M, N), torch.int16)
    fp8q.fp8q_gemm_rowscaled(dev(a), dev(km), dev(wq), dev(s_row), out.t, kernel=kernel)
    torch.cuda.synchronize()
    out.check_canary()
    return bf16_bits_to_f64(host(out.t))


def _row_operands(orc, M, N, K, seed, dist="normal"):
    rng = np.random.default_rng(seed)
    xf = rng.standard_normal((M, K)) if dist == "normal" else rng.laplace(0, 1, (M, K))
    x = synth.f32_to_bf16_bits(xf.astype(np.float32))
    a, a_s = orc.quant_act(x)
    wq, s_row = orc.quant_weight_row(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    return x, a, a_s, wq, s_row


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (16, 256, 512), (17, 384, 640), (64, 256, 1152),
                                   (130, 384, 640), (300, 512, 896)])
def test_gemm_rowscaled_small_full(orc, M, N, K):
    _, a, a_s, wq, s_row = _row_operands(orc, M, N, K, seed=M * 5 + N + K)
    ref = orc.gemm_ref(a, a_s, wq, s_row)
    for kern in _kernels_for(M):
        log(f"gemm_rowscaled M={M} N={N} K={K} kernel={kern}")
        assert_tol(_gemm_row_gpu(orc, a, a_s, wq, s_row, kern), ref, f"row M{M}N{N}K{K}k{kern}")


@pytest.mark.parametrize("M", [16, 25])
def test_gemm_rowscaled_decode_full(orc, M):
    w = synth.workload("decode", M=M)
    x, wf, _ = synth.make_inputs(w)
    a, a_s = orc.quant_act(x)
    wq, s_row = orc.quant_weight_row(wf)
    log(f"oracle rowscaled decode M={M}")
    ref = orc.gemm_ref(a, a_s, wq, s_row)
    for kern in _kernels_for(M):
        assert_tol(_gemm_row_gpu(orc, a, a_s, wq, s_row, kern), ref, f"row decode M{M} k{kern}")


@pytest.mark.slow
def test_gemm_rowscaled_large_prefill_full(orc):
    """Per-row weight scales at the large prefill size: all M*N outputs of the
    automatic, 128x128 and ping-pong kernels against the oracle."""
    w = synth.WORKLOADS["large_prefill"][0]
    x, wf, _ = synth.make_inputs(w)
    a, a_s = orc.quant_act(x)
    wq, s_row = orc.quant_weight_row(wf)
    log("oracle rowscaled large prefill: full fp64 product")
    ref = orc.gemm_ref(a, a_s, wq, s_row)
    for kern in (0, 1, 5):
        log(f"gemm_rowscaled large prefill kernel={kern}")
        assert_tol(_gemm_row_gpu(orc, a, a_s, wq, s_row, kern), ref, f"row large prefill k{kern}")


@pytest.mark.parametrize("M,N,K", [(300, 384, 1280), (2300, 384, 256)])
def test_gemm_rowscaled_tiled_bit_identical(orc, M, N, K):
    _, a, a_s, wq, s_row = _row_operands(orc, M, N, K, seed=7, dist="laplace")
    outs = {k: _gemm_row_gpu(orc, a, a_s, wq, s_row, k) for k in (1, 3, 4, 5, 0)}
    for k in (3, 4, 5, 0):
        assert np.array_equal(outs[k], outs[1]), f"kernel {k} differs from kernel 1"


def test_gemm_rowscaled_exact_cases(orc):
    """Codes 1.0 (0x38), power-of-two activation and row scales: every
    partial sum and product is exact, so the output is exact in bf16."""
    M, N, K = 48, 256, 384
    a = np.full((M, K), 0x38, dtype=np.uint8)
    wq = np.full((N, K), 0x38, dtype=np.uint8)
    rng = np.random.default_rng(2)
    a_s = np.ldexp(1.0, rng.integers(-6, 2, (M, K // 128))).astype(np.float32)
    s_row = np.ldexp(1.0, rng.integers(-6, 2, N)).astype(np.float32)
    ref = orc.gemm_ref(a, a_s, wq, s_row)
    for kern in _kernels_for(M):
        assert np.array_equal(_gemm_row_gpu(orc, a, a_s, wq, s_row, kern), ref), kern


@pytest.mark.parametrize("M,K", [(25, 5120), (3900, 17408)])
def test_proj_rowscaled_end_to_end(orc, M, K):
    N = 256
    x, a, a_s, wq, s_row = _row_operands(orc, M, N, K, seed=M + K, dist="laplace")
    assert fp8q.fp8q_proj_quant_fused(M, K) == (M * (K // 128) <= 1 << 19)
    ref = orc.gemm_ref(a, a_s, wq, s_row)
    out = Guarded((M, N), torch.int16)
    aq = Guarded((M, K), torch.uint8)
    asr = Guarded((M, K // 128), torch.float32)
    askm = Guarded((K // 128, synth.ceil16(M)), torch.float32, fill=0x7F)
    fp8q.fp8q_proj_rowscaled(dev(x), dev(wq), dev(s_row), out.t, aq.t, asr.t, askm.t)
    torch.cuda.synchronize()
    for g in (out, aq, asr, askm):
        g.check_canary()
    assert np.array_equal(host(aq.t), a)
    assert np.array_equal(host(askm.t).view(np.uint32), orc.scale_to_kmajor(a_s).view(np.uint32))
    assert_tol(bf16_bits_to_f64(host(out.t)), ref, f"proj_rowscaled M{M} K{K}")
