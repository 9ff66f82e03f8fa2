"""GPU parity of the bf16 comparator GEMM (fp8q_gemm_bf16): the bf16
projection act . W^T over the dequantized weight that the FP8 path is
measured against (page "dispatch_proj.rs").

* within the GEMM tolerance of the oracle's fp64 product at small sizes
  (full output, several tiles and a ragged last tile) and on the large
  prefill's dequantized weights (all outputs);
* exact on small-integer operands.
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


def _bf16_gpu(x, w):
    M, N = x.shape[0], w.shape[0]
    out = Guarded((M, N), torch.int16)
    fp8q.fp8q_gemm_bf16(dev(x.view(np.int16)), dev(w.view(np.int16)), out.t)
    torch.cuda.synchronize()
    out.check_canary()
    return bf16_bits_to_f64(host(out.t))


@pytest.mark.parametrize("M,N,K", [(1, 128, 64), (16, 256, 512), (300, 384, 1280), (600, 256, 192)])
def test_gemm_bf16_small_full(orc, M, N, K):
    rng = np.random.default_rng(M + N + K)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = synth.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    assert_tol(_bf16_gpu(x, w), orc.gemm_bf16_ref(x, w), f"bf16 M{M}N{N}K{K}")


def test_gemm_bf16_integer_exact(orc):
    rng = np.random.default_rng(3)
    xi = rng.integers(-4, 5, (70, 256))
    wi = rng.integers(-4, 5, (256, 256))
    x = synth.f32_to_bf16_bits(xi.astype(np.float32))
    w = synth.f32_to_bf16_bits(wi.astype(np.float32))
    # |sums| <= 4096: every output is an integer exact in fp32; compare
    # after the same bf16 rounding
    import oracle
    assert np.array_equal(_bf16_gpu(x, w), oracle.round_to_bf16(orc.gemm_bf16_ref(x, w)))


@pytest.mark.slow
def test_gemm_bf16_large_prefill_dequantized(orc):
    """The large prefill activations against its FP8 weights dequantized to
    bf16 by fp8q_dequant_fp8_bf16 (the comparator's real operands): all M*N
    outputs against the float64 product."""
    w = synth.WORKLOADS["large_prefill"][0]
    x, wf, _ = synth.make_inputs(w)
    wq, ws = orc.quant_weight_block(wf)
    wd = orc.dequant_fp8_bf16(wq, ws)
    out = _bf16_gpu(x, wd)
    log("oracle bf16 large prefill: full float64 product")
    assert_tol(out, orc.gemm_bf16_ref(x, wd), "bf16 large prefill")
