"""The divide-free scale and reciprocal of the quantizer kernels, checked in
exact arithmetic for every input they can meet.

The kernels form scale = fl32(amax / 448) and r = fl32(1 / scale) without a
divide (csrc/quant_common.h):

  scale = fma(-fma(q0, 448, -a), k, q0),  q0 = fl32(a * k),  k = fl32(1/448)
  r     = fma(fma(-scale, r0, 1), r0, r0),  r0 = the hardware reciprocal

Each fma is one rounding of the exact value, so every step is modelled here
with rational arithmetic and a single round-to-nearest-even to fp32.  The
first identity must hold for every finite bf16 magnitude a (the group
maximum is one); the second for every scale >= 2^-100 (smaller scales take
an exact divide) from any start r0 within one ulp of the correctly rounded
reciprocal, the accuracy of v_rcp_f32.  The quotients and codes built on
them are checked on the device for every (x, amax) pair by the exhaustive
quantizer test.
"""
from fractions import Fraction

import numpy as np

F_EMIN, F_MANT = -126, 23  # fp32: smallest normal exponent, stored mantissa bits


def round_f32(v: Fraction) -> float:
    """v rounded to the nearest fp32 value, ties to even (subnormals
    included; the values here stay far from overflow)."""
    if v == 0:
        return 0.0
    neg = v < 0
    v = -v if neg else v
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** e > v:
        e -= 1
    quantum = Fraction(2) ** (max(e, F_EMIN) - F_MANT)
    n = v / quantum
    whole = n.numerator // n.denominator
    rest = n - whole
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    r = float(whole * quantum)  # exact: an fp32 value is an fp64 value
    return -r if neg else r


def f32_bits(x: float) -> int:
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


def bits_f32(b: int) -> float:
    return float(np.array([b], dtype=np.uint32).view(np.float32)[0])


def test_round_f32_matches_numpy():
    rng = np.random.default_rng(5)
    for v in rng.standard_normal(2000) * np.exp2(rng.integers(-140, 100, 2000)):
        assert round_f32(Fraction(float(v))) == float(np.float32(v))


def test_scale_without_divide_every_bf16_magnitude():
    k = round_f32(Fraction(1, 448))
    assert k == float(np.float32(1) / np.float32(448))
    fk, f448 = Fraction(k), Fraction(448)
    for b in range(0x7F80):  # every finite bf16 magnitude, zero and subnormals included
        a = Fraction(bits_f32(b << 16))
        q0 = round_f32(a * fk)
        en = round_f32(Fraction(q0) * f448 - a)
        s = round_f32(Fraction(q0) - Fraction(en) * fk)
        ref = round_f32(a / f448)
        assert f32_bits(s) == f32_bits(ref), f"amax bits {b:#06x}"


def test_newton_reciprocal_every_scale():
    checked = 0
    for b in range(0x7F80):
        s = round_f32(Fraction(bits_f32(b << 16)) / 448)
        if not s >= 2.0 ** -100:
            continue
        fs = Fraction(s)
        rr = round_f32(1 / fs)
        for d in (-1, 0, 1):
            r0 = Fraction(bits_f32(f32_bits(rr) + d))
            e = round_f32(1 - fs * r0)
            r = round_f32(r0 + Fraction(e) * r0)
            assert r == rr, f"scale {s!r}, start {d:+d} ulp"
        checked += 1
    # maxima a >= 448 * 2^-100 = 1.75 * 2^-92: the top quarter of the binade
    # [2^-92, 2^-91) (32 values) and the 219 binades 2^-91 .. 2^127 (128 each)
    assert checked == 32 + 219 * 128
