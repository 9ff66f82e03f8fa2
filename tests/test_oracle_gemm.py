"""Pins of the oracle's block-scaled GEMM reference.

out[M,N] = act[M,K] . W[N,K]^T (page "dispatch_proj.rs", doc of
cublas_bf16_proj_dense for the orientation) with the activation scale of
(m, kb) and the weight scale of the 128x128 block (n/128, kb) applied per
128-deep K block (doc of cublas_fp8_proj; weight-scale index from
dequant_fp8_bf16_into).

* library routine: equals numpy's float64 matmul of the dequantized operands;
* closed forms: block-scale isolation (all codes 1.0, power-of-two scales
  that differ per row, per K block and per N block) and one-hot weight rows;
* the sampled entry point agrees with the full one;
* the error metric: bf16 ulp closed form and behaviour on known offsets.
"""
import numpy as np
import pytest

import synth


def _dequant_act(orc, a, a_s):
    M, K = a.shape
    return orc.e4m3_decode(a) * np.repeat(a_s.astype(np.float64), 128, axis=1)


def _dequant_w(orc, w, w_s):
    return orc.e4m3_decode(w) * np.repeat(np.repeat(w_s.astype(np.float64), 128, axis=0), 128, axis=1)


def _random_operands(orc, M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a, a_s = orc.quant_act(x)
    w, w_s = orc.quant_weight_block(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    return a, a_s, w, w_s


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (16, 256, 512), (37, 384, 640)])
def test_matches_numpy_dgemm(orc, M, N, K):
    a, a_s, w, w_s = _random_operands(orc, M, N, K, seed=M + N + K)
    ref = orc.gemm_ref(a, a_s, w, w_s)
    lib = _dequant_act(orc, a, a_s) @ _dequant_w(orc, w, w_s).T
    assert np.max(np.abs(ref - lib)) <= 1e-12 * np.max(np.abs(lib))


def test_block_scale_isolation_closed_form(orc):
    M, N, K = 20, 384, 768
    G = K // 128
    a = np.full((M, K), 0x38, dtype=np.uint8)            # 1.0
    w = np.full((N, K), 0x38, dtype=np.uint8)
    a_s = np.array([[2.0 ** (m % 5) for _ in range(G)] for m in range(M)], dtype=np.float32)
    w_s = np.array([[2.0 ** g * (nb + 1) for g in range(G)] for nb in range(N // 128)],
                   dtype=np.float32)
    ref = orc.gemm_ref(a, a_s, w, w_s)
    for m in range(M):
        for n in range(0, N, 7):
            want = 128.0 * sum(2.0 ** (m % 5 + g) * (n // 128 + 1) for g in range(G))
            assert ref[m, n] == want


def test_one_hot_weight_rows(orc):
    M, N, K = 9, 256, 512
    G = K // 128
    rng = np.random.default_rng(11)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a, a_s = orc.quant_act(x)
    kk = rng.integers(0, K, size=N)
    w = np.zeros((N, K), dtype=np.uint8)
    w[np.arange(N), kk] = 0x38
    w_s = rng.uniform(0.5, 2.0, (N // 128, G)).astype(np.float32)
    ref = orc.gemm_ref(a, a_s, w, w_s)
    dec = orc.e4m3_decode(a)
    for n in range(N):
        k = kk[n]
        want = dec[:, k] * a_s[:, k // 128].astype(np.float64) * float(w_s[n // 128, k // 128])
        assert np.array_equal(ref[:, n], want)


def test_sampled_matches_full(orc):
    M, N, K = 23, 256, 384
    a, a_s, w, w_s = _random_operands(orc, M, N, K, seed=5)
    ref = orc.gemm_ref(a, a_s, w, w_s)
    rng = np.random.default_rng(0)
    ms = rng.integers(0, M, 500)
    ns = rng.integers(0, N, 500)
    assert np.array_equal(orc.gemm_ref_at(a, a_s, w, w_s, ms, ns), ref[ms, ns])


def test_transposed_scale_is_caught(orc):
    """A plausible mistake in the reference -- the K-major activation scale read
    as if it were row-major -- moves the result far outside the tolerance."""
    M, N, K = 16, 256, 1024
    a, a_s, w, w_s = _random_operands(orc, M, N, K, seed=9)
    ref = orc.gemm_ref(a, a_s, w, w_s)
    km = orc.scale_to_kmajor(a_s)                        # [G, 16]
    wrong = np.ascontiguousarray(km.ravel()[: M * (K // 128)].reshape(M, K // 128))
    bad = orc.gemm_ref(a, wrong, w, w_s)
    rel, exc, _ = orc.gemm_errors(bad, ref)
    assert rel > 1e-2 and exc > 10


def test_bf16_ulp_and_metric(orc):
    r = np.array([1.0, 1.5, 2.0, -3.0, 2.0 ** -126, 2.0 ** -130, 0.0])
    want = np.array([2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -133, 2.0 ** -133, 2.0 ** -133])
    assert np.array_equal(orc.bf16_ulp(r), want)
    ref = np.linspace(-4, 4, 1001)
    rel, exc, relf = orc.gemm_errors(orc.round_to_bf16(ref), ref)
    assert rel == 0 and exc <= 0.5 / (1 + 1e-12) + 1e-12 and relf > 0
    rms = float(np.sqrt(np.mean(ref * ref)))
    off = ref + (orc.bf16_ulp(ref) + 1e-3 * rms) * 0.999
    rel, exc, _ = orc.gemm_errors(off, ref)
    assert exc < 1.0
    off = ref + (orc.bf16_ulp(ref) + 1e-3 * rms) * 1.01
    assert orc.gemm_errors(off, ref)[1] > 1.0


def test_round_to_bf16_matches_torch_and_ties(orc):
    import torch
    rng = np.random.default_rng(6)
    v = (rng.standard_normal(200_000) * np.exp2(rng.integers(-40, 40, 200_000))).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.round_to_bf16(v.astype(np.float64)), want)
    # fp64 values just off a bf16 midpoint round by the sign of the offset
    # (a detour through fp32 would lose the offset and tie to even)
    lo = np.float64(1.0)
    mid = lo + 2.0 ** -8                       # halfway between 1 and 1 + 2^-7
    assert orc.round_to_bf16(np.array([mid]))[0] == 1.0            # tie -> even
    assert orc.round_to_bf16(np.array([mid + 2.0 ** -40]))[0] == 1.0 + 2.0 ** -7
    assert orc.round_to_bf16(np.array([mid - 2.0 ** -40]))[0] == 1.0
    assert orc.round_to_bf16(np.array([-(mid + 2.0 ** -40)]))[0] == -(1.0 + 2.0 ** -7)


def test_bf16_output_rounding_floor(orc):
    """Rounding an exact result to bf16 alone gives a relative RMS error of
    about 1.66e-3 (uniform rounding error of 2^-7 relative ulp), which is why
    the 1e-3 relative-RMS bar is applied against the bf16-rounded reference."""
    rng = np.random.default_rng(1)
    r = rng.standard_normal(400_000) * 3.0
    _, _, relf = orc.gemm_errors(orc.round_to_bf16(r), r)
    assert 1.5e-3 < relf < 1.8e-3
