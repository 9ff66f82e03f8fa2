"""Seeded shape fuzz of the block-scaled GEMM: random (M, N, K) with ragged
row counts (1 .. 700), column counts of 1 .. 10 weight blocks and 1 .. 24 K
blocks, random activation magnitudes per row, through every kernel the API
can force and the split-K form at a random split count, each against the
oracle's fp64 product with the projection tolerance (rel_rms <= 1e-3 against
the bf16-rounded reference; per element <= 1 bf16 ulp + 1e-3 * RMS).  The
tiled kernels must agree bit for bit with each other as well."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import Guarded, bf16_bits_to_f64, dev, host, log, require_gpu

pytestmark = pytest.mark.gpu

fp8q = None
RTOL = 1e-3
N_CASES = 24


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global fp8q
    require_gpu()
    import w8a8_fp8_block_amd as m
    fp8q = m
    yield


def _case(i):
    rng = np.random.default_rng(1000 + i)
    M = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 300)),
                        int(rng.integers(300, 701))]))
    N = 128 * int(rng.integers(1, 11))
    K = 128 * int(rng.integers(1, 25))
    return rng, M, N, K


@pytest.mark.parametrize("i", range(N_CASES))
def test_gemm_shape_fuzz(orc, i):
    rng, M, N, K = _case(i)
    x = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-4, 4, (M, 1)))).astype(np.float32)
    x_bits = synth.f32_to_bf16_bits(x)
    a, a_s = orc.quant_act(x_bits)
    wq, ws = orc.quant_weight_block(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    km = orc.scale_to_kmajor(a_s)
    ref = orc.gemm_ref(a, a_s, wq, ws)
    ad, kmd, wd, wsd = dev(a), dev(km), dev(wq), dev(ws)
    outs = {}
    for kern in (0, 1, 2, 3, 4, 5):
        log(f"fuzz {i}: M={M} N={N} K={K} kernel={kern}")
        out = Guarded((M, N), torch.int16)
        fp8q.fp8q_gemm_blockscaled(ad, kmd, wd, wsd, out.t, kernel=kern)
        torch.cuda.synchronize()
        out.check_canary()
        outs[kern] = bf16_bits_to_f64(host(out.t))
    G = K // 128
    if G >= 2:
        splits = int(rng.integers(2, min(G, 12) + 1))
        log(f"fuzz {i}: split-K splits={splits}")
        need = fp8q.fp8q_gemm_splitk_workspace_bytes(M, N, K, splits)
        work = Guarded((need // 4,), torch.float32, fill=0x7F)
        out = Guarded((M, N), torch.int16)
        fp8q.fp8q_gemm_blockscaled_splitk(ad, kmd, wd, wsd, out.t, work.t, splits=splits)
        torch.cuda.synchronize()
        out.check_canary()
        work.check_canary()
        outs["splitk"] = bf16_bits_to_f64(host(out.t))
    for k, o in outs.items():
        rel, exc, _ = orc.gemm_errors(o, ref)
        assert rel <= RTOL and exc <= 1.0, f"case {i} (M={M} N={N} K={K}) kernel {k}: rel {rel} exc {exc}"
    for k in (3, 4, 5):
        assert np.array_equal(outs[k], outs[1]), f"case {i}: kernel {k} differs from kernel 1"
