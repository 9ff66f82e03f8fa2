"""Pins of the oracle's FFN-chain functions.

Page "dispatch_proj.rs", doc of cublas_fp8_proj_prequant: the dense FFN's
gate and up projections read the same [M,K] input, which is quantized once
for both; the post-SiLU intermediate is quantized once for the down
projection.  The oracle's reading: h = bf16(silu(gate) * up) with
silu(g) = g / (1 + e^-g), each projection's output bf16.

* ``f64_to_bf16``: equal to torch's fp32 -> bf16 cast wherever the value is
  an fp32 number (one rounding either way); one rounding, not two, for values
  just off a bf16 midpoint; ties to even; overflow to infinity;
* ``silu_mul``: equal to the bf16 rounding of torch's float64 SiLU times up;
  closed forms (zero gate, large positive and negative gates, the gate/up
  order); the identity silu(-g) = silu(g) - g; every element where a float32
  evaluation (torch's) rounds differently lies in the reported ambiguity
  mask;
* ``ffn_ref``: the whole chain against an independent brute-force chain of
  pure-Python loops (search encoder, math.exp, search rounding to bf16) on a
  tiny shape with H != I, and row restriction equal to the full result's
  rows.
"""
import math

import numpy as np
import pytest
import torch

import brute
import synth


def _t_bits(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _all_finite_bf16(rng, n):
    b = rng.integers(0, 1 << 16, n, dtype=np.int64).astype(np.uint16)
    return b[(b & 0x7F80) != 0x7F80]


# ------------------------------------------------------------ f64_to_bf16
def test_f64_to_bf16_equals_torch_cast_on_fp32_values(orc):
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 32, 400_000, dtype=np.int64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.38e38)]
    ours = orc.f64_to_bf16(f.astype(np.float64))
    assert np.array_equal(ours, _t_bits(torch.from_numpy(f)))


def test_f64_to_bf16_single_rounding_ties_and_overflow(orc):
    # 1 + 2^-8 is the midpoint between bf16 1.0 and 1 + 2^-7: ties to even
    # (1.0); a double just above it must round up although its fp32
    # rounding is the midpoint itself (two roundings would give 1.0).
    one_up = 1.0 + 2.0 ** -7
    cases = {
        1.0 + 2.0 ** -8: 1.0,
        1.0 + 2.0 ** -8 + 2.0 ** -40: one_up,
        1.0 + 2.0 ** -8 - 2.0 ** -40: 1.0,
        one_up + 2.0 ** -8: 1.0 + 2.0 ** -6,  # tie between odd and even: to even (up)
        -(1.0 + 2.0 ** -8 + 2.0 ** -40): -one_up,
        2.0 ** -134: 0.0,  # half the smallest subnormal: tie to even zero
        2.0 ** -134 + 2.0 ** -160: 2.0 ** -133,
        3.0 * 2.0 ** -134: 2.0 ** -132,  # 1.5 subnormal ulps: tie to even (2 ulps)
        (2.0 - 2.0 ** -7) * 2.0 ** 127: (2.0 - 2.0 ** -7) * 2.0 ** 127,  # bf16 max
        (2.0 - 2.0 ** -8) * 2.0 ** 127: math.inf,  # max + half ulp: tie to 2^128
        (2.0 - 2.0 ** -8) * 2.0 ** 127 - 2.0 ** 100: (2.0 - 2.0 ** -7) * 2.0 ** 127,
    }
    v = np.array(list(cases.keys()), dtype=np.float64)
    want = np.array(list(cases.values()), dtype=np.float64)
    got = orc.bf16_to_f64(orc.f64_to_bf16(v))
    assert np.array_equal(got, want), np.stack([v, got, want], 1)
    z = orc.f64_to_bf16(np.array([0.0, -0.0, -2.0 ** -140]))
    assert list(z) == [0x0000, 0x8000, 0x8000]


# --------------------------------------------------------------- silu_mul
def test_silu_mul_equals_torch_float64(orc):
    rng = np.random.default_rng(12)
    g = _all_finite_bf16(rng, 300_000)
    g = g[np.abs(orc.bf16_to_f64(g)) < 200.0]
    u = _all_finite_bf16(rng, g.size)
    u = u[:g.size]
    g = g[:u.size]
    h, _ = orc.silu_mul(g, u)
    gv, uv = torch.from_numpy(orc.bf16_to_f64(g)), torch.from_numpy(orc.bf16_to_f64(u))
    ref = (torch.nn.functional.silu(gv) * uv).numpy()
    assert np.array_equal(h, orc.f64_to_bf16(ref))


def test_silu_mul_closed_forms(orc):
    def bf(vals):
        return synth.f32_to_bf16_bits(np.array(vals, dtype=np.float32))

    # zero gate: silu(0) = 0, the sign follows up
    h, _ = orc.silu_mul(bf([0.0, 0.0]), bf([3.0, -3.0]))
    assert list(h) == [0x0000, 0x8000]
    # large positive gates: silu(g) = g (1 - e^-g), e^-g far below half a bf16 ulp
    g = bf(np.linspace(64.0, 3.0e4, 257))
    h, amb = orc.silu_mul(g, bf(np.ones(257)))
    assert np.array_equal(h, g) and not amb.any()
    # large negative gate: |silu(g)| = |g| e^g < 2^-134, rounds to -0
    h, _ = orc.silu_mul(bf([-100.0, -1000.0]), bf([1.0, 1.0]))
    assert list(h) == [0x8000, 0x8000]
    # gate/up order: silu(-2) * 3 = -6 / (1 + e^2) = -0.7152...; bf16 ulp in
    # [0.5, 1) is 2^-8, -0.7152 * 256 = -183.09 -> -183/256.  (Swapped, the
    # value would be silu(3) * -2 = -5.715.)
    h, _ = orc.silu_mul(bf([-2.0]), bf([3.0]))
    assert orc.bf16_to_f64(h)[0] == -183.0 / 256.0


def test_silu_mul_reflection_identity(orc):
    # silu(-g) = -g (1 - sigma(g)) = silu(g) - g
    rng = np.random.default_rng(13)
    g = synth.f32_to_bf16_bits(rng.normal(0.0, 4.0, 50_000).astype(np.float32))
    u = synth.f32_to_bf16_bits(rng.normal(0.0, 2.0, 50_000).astype(np.float32))
    neg = g ^ np.uint16(0x8000)
    h_neg, _ = orc.silu_mul(neg, u)
    gv, uv = orc.bf16_to_f64(g), orc.bf16_to_f64(u)
    sig = 1.0 / (1.0 + np.exp(-gv))
    want = orc.f64_to_bf16((gv * sig - gv) * uv)
    # two float64 evaluations of one value: equal unless within ~1e-15 of a
    # rounding midpoint
    diff = h_neg != want
    assert diff.sum() <= 2, diff.sum()


def test_silu_mul_ambiguity_mask_covers_float32_evaluation(orc):
    rng = np.random.default_rng(14)
    g = synth.f32_to_bf16_bits(rng.normal(0.0, 3.0, 400_000).astype(np.float32))
    u = synth.f32_to_bf16_bits(rng.normal(0.0, 2.0, 400_000).astype(np.float32))
    h, amb = orc.silu_mul(g, u)
    g32 = torch.from_numpy(synth.bf16_bits_to_f32(g))
    u32 = torch.from_numpy(synth.bf16_bits_to_f32(u))
    h32 = _t_bits(torch.nn.functional.silu(g32) * u32)
    differs = h32 != h
    assert not (differs & ~amb).any(), int((differs & ~amb).sum())
    assert amb.mean() < 0.01  # the band is narrow: about 2^-9 of elements


# ------------------------------------------------------------------ chain
def _brute_bf16(v: float) -> int:
    """bf16 bits of the double v by search: the two bf16 neighbours around the
    fp32 rounding of v, nearest chosen in exact double arithmetic, ties to the
    even pattern."""
    f = np.array([v], dtype=np.float32)
    b = int(f.view(np.uint32)[0] >> 16)
    cands = {b, (b + 1) & 0xFFFF, (b - 1) & 0xFFFF}
    best, bestd = None, None
    for c in sorted(cands):
        cv = brute.bf16_value(c)
        if math.isnan(cv) or math.copysign(1.0, cv) != math.copysign(1.0, v):
            if not (v == 0.0 and cv == 0.0):
                continue
        d = abs(cv - v)
        if bestd is None or d < bestd or (d == bestd and (c & 1) == 0):
            best, bestd = c, d
    return best


def _brute_gemm(codes_a, s_a, codes_w, s_w):
    """Block form with numpy float64 dot products (one per 128-deep block)."""
    M, K = codes_a.shape
    N = codes_w.shape[0]
    va = np.array(brute.VALUES)[codes_a]
    vw = np.array(brute.VALUES)[codes_w]
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for g in range(K // 128):
                S = float(np.dot(va[m, 128 * g:128 * (g + 1)], vw[n, 128 * g:128 * (g + 1)]))
                acc += float(s_a[m, g]) * float(s_w[n // 128, g]) * S
            out[m, n] = acc
    return out


def test_ffn_ref_against_brute_force_chain(orc):
    M, H, I = 3, 256, 384
    w = synth.FfnWorkload("t", M, H, I, 1, 20.0, seed=21)
    x, (wg, wu, wd) = synth.make_ffn_inputs(w)
    (gq, gs), (uq, us), (dq, ds) = (orc.quant_weight_block(a) for a in (wg, wu, wd))
    ref = orc.ffn_ref(x, gq, gs, uq, us, dq, ds)

    xq, xs = brute.quant_act(x)
    g = _brute_gemm(xq, xs, gq, gs)
    u = _brute_gemm(xq, xs, uq, us)
    gb = np.array([[_brute_bf16(v) for v in r] for r in g], dtype=np.uint16)
    ub = np.array([[_brute_bf16(v) for v in r] for r in u], dtype=np.uint16)
    hv = [[brute.bf16_value(int(a)) / (1.0 + math.exp(-brute.bf16_value(int(a))))
           * brute.bf16_value(int(b)) for a, b in zip(ra, rb)] for ra, rb in zip(gb, ub)]
    hb = np.array([[_brute_bf16(v) for v in r] for r in hv], dtype=np.uint16)
    hq, hs = brute.quant_act(hb)
    out = _brute_gemm(hq, hs, dq, ds)

    assert np.array_equal(ref["xq"], xq) and np.array_equal(ref["xs"], xs)
    assert np.array_equal(ref["g"], gb) and np.array_equal(ref["u"], ub)
    assert np.array_equal(ref["h"], hb)
    assert np.array_equal(ref["hq"], hq) and np.array_equal(ref["hs"], hs)
    assert ref["out"].shape == (M, H)
    np.testing.assert_allclose(ref["out"], out, rtol=1e-12, atol=1e-12 * np.abs(out).max())


def test_ffn_ref_rows_restriction(orc):
    w = synth.ffn_workload("ffn_tiny")
    x, (wg, wu, wd) = synth.make_ffn_inputs(w)
    (gq, gs), (uq, us), (dq, ds) = (orc.quant_weight_block(a) for a in (wg, wu, wd))
    full = orc.ffn_ref(x, gq, gs, uq, us, dq, ds)
    rows = [0, 5, 15]
    part = orc.ffn_ref(x, gq, gs, uq, us, dq, ds, rows=rows)
    for k in ("xq", "xs", "g", "u", "h", "hq", "hs", "out"):
        assert np.array_equal(part[k], full[k][rows]), k
