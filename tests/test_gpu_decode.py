"""GPU parity of the decode-width GEMM (up to 64 rows: the automatic
choice, kernel id 2) against the oracle's fp64 block-form product, all M*N
outputs, within the GEMM tolerance.  Two kernels sit behind it: the one
whose per-workgroup weight slice is loaded into LDS in one go (up to 32
rows and 32 columns a workgroup and 48 K blocks: N = 6144, K = 5120 on one
workgroup per CU), and the fragment-layout one for the rest.  The shapes
cover, for the first: one and two 16-row tiles (M = 3, 16, 20, 25, 32),
ranges of one and of one and a half 16-column tiles, ranges of unequal width
(N = 5248: 1312 four-column units over the workgroups), K ending in a
partial 1 KB row piece (K = 1280, 2176); for the second: up to 64 rows and
wider ranges (N = 10240 .. 32768), 48-row tiles (M = 40, 45: three 16-row
tiles), and beyond 64 rows (M = 100: two 64-row tiles, 64 columns a
workgroup); between them every wave count the skinny kernel takes (8 waves
at two, three and four row tiles with up to eight column tiles where their
partial sums fit in 128 KB, 4 beyond: M = 45, N = 17408).  Both
weight-scale formats throughout.
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


def _operands(orc, M, N, K, seed, per_row=False):
    rng = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits(rng.laplace(0, 1, (M, K)).astype(np.float32))
    a, a_s = orc.quant_act(x)
    wf = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    wq, ws = orc.quant_weight_row(wf) if per_row else orc.quant_weight_block(wf)
    return a, a_s, wq, ws


def _run(orc, a, a_s, wq, ws, per_row):
    M, K = a.shape
    N = wq.shape[0]
    out = Guarded((M, N), torch.int16)
    km = dev(orc.scale_to_kmajor(a_s))
    gemm = fp8q.fp8q_gemm_rowscaled if per_row else fp8q.fp8q_gemm_blockscaled
    gemm(dev(a), km, dev(wq), dev(ws), out.t, kernel=2)
    torch.cuda.synchronize()
    out.check_canary()
    return bf16_bits_to_f64(host(out.t))


CASES = [(3, 6144, 1280), (16, 5248, 2048), (32, 6144, 3072), (17, 4096, 5120),
         (25, 6144, 5120), (25, 17408, 1152), (64, 6144, 5120), (16, 32768, 512),
         (40, 10240, 2176), (64, 20480, 384), (25, 28672, 1024), (100, 6144, 2048),
         (45, 17408, 5120)]


@pytest.mark.parametrize("per_row", [False, True], ids=["block", "row"])
@pytest.mark.parametrize("M,N,K", CASES, ids=[f"M{m}N{n}K{k}" for m, n, k in CASES])
def test_decode_kernel_full(orc, M, N, K, per_row):
    assert fp8q.fp8q_gemm_select(M, N, K) == 2
    a, a_s, wq, ws = _operands(orc, M, N, K, M + N + K, per_row)
    log(f"oracle decode M={M} N={N} K={K} per_row={per_row}")
    ref = orc.gemm_ref(a, a_s, wq, ws)
    log(f"decode kernel M={M} N={N} K={K} per_row={per_row}")
    o1 = _run(orc, a, a_s, wq, ws, per_row)
    assert_tol(o1, ref, f"decode M{M}N{N}K{K} row={per_row}")
    o2 = _run(orc, a, a_s, wq, ws, per_row)
    assert np.array_equal(o1, o2), "not repeatable"


def test_decode_kernel_exact(orc):
    """Codes 1.0 and power-of-two scales, 17 K blocks (a partial last stage)
    and unequal column ranges: every partial sum is exact, so the output is
    the oracle's value rounded to bf16, bit for bit."""
    M, N, K = 20, 5248, 17 * 128
    a = np.full((M, K), 0x38, dtype=np.uint8)
    wq = np.full((N, K), 0x38, dtype=np.uint8)
    rng = np.random.default_rng(8)
    a_s = np.ldexp(1.0, rng.integers(-6, 2, (M, K // 128))).astype(np.float32)
    ws = np.ldexp(1.0, rng.integers(-6, 2, (N // 128, K // 128))).astype(np.float32)
    got = _run(orc, a, a_s, wq, ws, False)
    assert np.array_equal(got, orc.round_to_bf16(orc.gemm_ref(a, a_s, wq, ws)))
