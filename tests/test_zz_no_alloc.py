"""GPU check of fp8q_gemm_blockscaled_splitk_noalloc, the split-K GEMM entry
point that keeps its fp32 partials in the library's static device scratch
(for callers that cannot allocate), called through the raw C ABI.

Two calls in a row, the second with a smaller input (the scratch keeps the
first call's contents), each compared bit for bit with
fp8q_gemm_blockscaled_splitk (same kernels, caller workspace, same split
count) and with the oracle to the GEMM tolerance; output canaries on both
sides.  A size past the scratch is refused before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import Guarded, assert_tol, bf16_bits_to_f64, dev, host, log, require_gpu

pytestmark = pytest.mark.gpu


def _operands(orc, M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits(rng.laplace(0, 1, (M, K)).astype(np.float32))
    a, a_s = orc.quant_act(x)
    wq, ws = orc.quant_weight_block(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    return a, a_s, wq, ws


def test_noalloc_splitk_matches_the_workspace_entry(orc):
    require_gpu()
    import w8a8_fp8_block_amd as fp8q
    L = fp8q.lib()
    stream = torch.cuda.current_stream().cuda_stream
    # (M, N, K, splits): the first fills 31.5 MB of the 32 MiB scratch with
    # the automatic count (3); the second is smaller, with a forced count;
    # the third, smaller again, runs the skinny kernel's split form (48 rows)
    for M, N, K, splits in ((512, 5120, 17408, 0), (200, 1024, 5120, 3), (48, 5120, 17408, 0)):
        a, a_s, wq, ws = _operands(orc, M, N, K, M + N)
        eff = splits or fp8q.fp8q_gemm_splitk_select(M, N, K)
        assert eff >= 2
        assert eff * M * N * 4 <= fp8q.NOALLOC_SCRATCH_BYTES
        log(f"noalloc splitk M={M} N={N} K={K} splits={splits} (runs {eff})")
        ad, kmd, wqd, wsd = dev(a), dev(orc.scale_to_kmajor(a_s)), dev(wq), dev(ws)
        out = Guarded((M, N), torch.int16)
        st = L.fp8q_gemm_blockscaled_splitk_noalloc(ad.data_ptr(), kmd.data_ptr(), wqd.data_ptr(),
                                                    wsd.data_ptr(), out.t.data_ptr(), M, N, K,
                                                    splits, ctypes.c_void_p(stream))
        assert st == 0, fp8q.lib().fp8q_last_error().decode()
        torch.cuda.synchronize()
        out.check_canary()
        got = host(out.t)
        # the entry point with a caller workspace, same split count
        need = fp8q.fp8q_gemm_splitk_workspace_bytes(M, N, K, eff)
        ref_out = Guarded((M, N), torch.int16)
        work = torch.empty((need // 4,), dtype=torch.float32, device="cuda")
        fp8q.fp8q_gemm_blockscaled_splitk(ad, kmd, wqd, wsd, ref_out.t, work, splits=eff)
        torch.cuda.synchronize()
        ref_out.check_canary()
        assert np.array_equal(got, host(ref_out.t)), "differs from the workspace entry point"
        log(f"oracle M={M} N={N} K={K}")
        assert_tol(bf16_bits_to_f64(got), orc.gemm_ref(a, a_s, wq, ws), f"noalloc M{M}N{N}K{K}")


def test_noalloc_splitk_refuses_sizes_past_the_scratch():
    require_gpu()
    import w8a8_fp8_block_amd as fp8q
    L = fp8q.lib()
    buf = torch.empty(256, dtype=torch.uint8, device="cuda")
    p = buf.data_ptr()
    # 3 * 600 * 5120 * 4 bytes = 36.9 MB > 32 MiB: refused before any launch,
    # so the placeholder pointers are never read
    st = L.fp8q_gemm_blockscaled_splitk_noalloc(p, p, p, p, p, 600, 5120, 17408, 3, None)
    assert st == 2
    assert "static scratch" in L.fp8q_last_error().decode()
