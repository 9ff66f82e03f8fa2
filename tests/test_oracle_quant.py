"""Pins of the oracle's activation quantizer and scale relayout.

* brute force: an independent pure-Python implementation (tests/brute.py)
  agrees bit-exactly on tiny inputs, including hand-made groups;
* exhaustive element map: for every finite (x, amax) bf16 pair, |x| <= amax,
  the oracle's code equals numpy's IEEE fp32 quotient encoded by PyTorch's
  float8_e4m3fn cast (library routines);
* the invariants of the method: each group's amax element encodes to +-448,
  K-major pad slots are zero, the relayout is a bijection onto the non-pad
  slots; plus sign preservation, no NaN codes, monotone decode and the
  half-ulp error bound.

Layouts follow the page "dispatch_proj.rs": scales [M, K/128] row-major from
the quantizer (doc of cublas_fp8_proj), K-major [K/128, ceil16(M)] with the
pad rows zero (docs of cublas_scale_layout_kmajor, fp8_act_scale_to_kmajor
and cublas_fp8_m_pad).
"""
import numpy as np
import pytest
import torch

import brute
import synth
from synth import bf16_bits_to_f32, f32_to_bf16_bits


def _handmade_groups() -> np.ndarray:
    """Rows of 128 bf16 patterns exercising the corner cases."""
    rows = []
    z = np.zeros(128, dtype=np.uint16)
    rows.append(z.copy())                                 # all +0
    r = z.copy(); r[::2] = 0x8000; rows.append(r)         # +0 / -0 mix
    r = z.copy(); r[5] = f32_to_bf16_bits(np.array([-3.5], np.float32))[0]; rows.append(r)  # single nonzero
    r = z.copy(); r[0] = 0x0001; r[1] = 0x8001; rows.append(r)  # smallest subnormal amax
    r = z.copy(); r[:] = np.arange(128, dtype=np.uint16) + 0x0010; rows.append(r)  # subnormal group
    r = z.copy(); r[:] = 0x0080 + np.arange(128, dtype=np.uint16); rows.append(r)  # near 2^-126
    # ties in amax: several elements at +-amax
    v = np.linspace(-1, 1, 128).astype(np.float32); v[3] = 7.0; v[9] = -7.0; v[100] = 7.0
    rows.append(f32_to_bf16_bits(v))
    # exact e4m3 midpoints relative to amax = 448 (scale 1.0)
    mids = np.array([0.5 * (a + b) for a, b in zip(range(0, 64, 2), range(1, 65, 2))] * 4,
                    dtype=np.float32)[:128] / 8.0
    mids[0] = 448.0
    rows.append(f32_to_bf16_bits(mids))
    # large magnitudes near the bf16 maximum
    r = np.full(128, 0x7F7F, dtype=np.uint16); r[1::2] = 0xFF00; rows.append(r)
    return np.stack(rows)


def test_brute_force_tiny_random(orc):
    rng = np.random.default_rng(7)
    for M, K in ((1, 128), (3, 256), (4, 512)):
        x = f32_to_bf16_bits((rng.standard_normal((M, K)) *
                              np.exp(rng.uniform(-30, 30, (M, 1)))).astype(np.float32))
        q, s = orc.quant_act(x)
        bq, bs = brute.quant_act(x)
        assert np.array_equal(s.view(np.uint32), bs.view(np.uint32))
        assert np.array_equal(q, bq)


def test_brute_force_handmade(orc):
    x = _handmade_groups().reshape(1, -1)
    q, s = orc.quant_act(x)
    bq, bs = brute.quant_act(x)
    assert np.array_equal(s.view(np.uint32), bs.view(np.uint32))
    assert np.array_equal(q, bq)
    # the zero groups: scale +0, codes keep the sign of zero
    assert s[0, 0] == 0 and s[0, 1] == 0
    assert np.all(q[0, :128] == 0)
    assert np.all(q[0, 128:256][::2] == 0x80) and np.all(q[0, 128:256][1::2] == 0)


def test_scale_closed_form(orc):
    w = synth.workload("tiny")
    x, _, _ = synth.make_inputs(w, with_weights=False)
    _, s = orc.quant_act(x)
    xf = bf16_bits_to_f32(x).reshape(w.M, -1, 128)
    amax = np.abs(xf).max(axis=2)
    assert np.array_equal(s.view(np.uint32), (amax / np.float32(448.0)).astype(np.float32).view(np.uint32))


def _check_invariants(orc, x, q, s):
    M, K = x.shape
    G = K // 128
    xf = bf16_bits_to_f32(x).reshape(M, G, 128)
    qg = q.reshape(M, G, 128)
    # no NaN codes
    assert not np.any((q & 0x7F) == 0x7F)
    # sign preserved (including signed zero)
    assert np.array_equal(qg >> 7, (x.reshape(M, G, 128) >> 15).astype(np.uint8))
    # I1: every element with |x| == amax (amax > 0) encodes to +-448
    amax = np.abs(xf).max(axis=2, keepdims=True)
    hit = (np.abs(xf) == amax) & (amax > 0)
    assert np.all((qg[hit] & 0x7F) == 0x7E)
    # monotone: |x| ordering is never reversed by the codes within a group
    dec = np.abs(orc.e4m3_decode(qg))
    ax = np.abs(xf)
    for m in range(min(M, 4)):
        for g in range(min(G, 8)):
            order = np.argsort(ax[m, g], kind="stable")
            assert np.all(np.diff(dec[m, g][order]) >= 0)
    # error bound: |dec*s - x| <= (1/2 ulp_e4m3(q) + 1/2 ulp_f32(q)) * s
    sf = s.reshape(M, G, 1).astype(np.float64)
    nz = sf[..., 0] > 0
    qv = np.where(sf > 0, xf / np.where(sf > 0, sf, 1), 0)
    aq = np.abs(qv)
    e = np.floor(np.log2(np.maximum(aq, 2.0 ** -6)))
    ulp8 = np.ldexp(1.0, (e - 3).astype(np.int64))
    ulp32 = np.ldexp(1.0, (np.floor(np.log2(np.maximum(aq, 2.0 ** -126))) - 23).astype(np.int64))
    err = np.abs(orc.e4m3_decode(qg) * sf - xf)
    bound = (0.5 * ulp8 + 0.5 * ulp32) * sf
    assert np.all(err[nz] <= bound[nz] * (1 + 1e-12))


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_invariants_on_workloads(orc, name):
    for w in synth.WORKLOADS[name]:
        x, _, _ = synth.make_inputs(w, with_weights=False)
        q, s = orc.quant_act(x)
        _check_invariants(orc, x, q, s)


def test_invariants_on_laplace_outliers(orc):
    w = synth.workload("large_prefill")
    x, _, _ = synth.make_inputs(w, M=24, with_weights=False)
    q, s = orc.quant_act(x)
    _check_invariants(orc, x, q, s)


@pytest.mark.parametrize("M", [1, 15, 16, 17, 25, 33])
def test_relayout_bijection_and_pad(orc, M):
    K = 640
    rng = np.random.default_rng(M)
    rm = rng.random((M, K // 128), dtype=np.float32) + 0.5
    km = orc.scale_to_kmajor(rm)
    Mp = synth.ceil16(M)
    assert km.shape == (K // 128, Mp)
    # I2 pad slots are +0.0 (all bits zero)
    assert np.all(km[:, M:].view(np.uint32) == 0)
    # I3 km[g, m] == rm[m, g] for m < M, and each real slot is hit once
    assert np.array_equal(km[:, :M], rm.T)
    assert np.array_equal(km, brute.kmajor(rm))
    flat = km.ravel()
    hit = np.zeros(rm.size, dtype=np.int64)
    idx = {v: i for i, v in enumerate(rm.ravel().tolist())}
    if len(idx) == rm.size:  # distinct values: check the bijection directly
        for v in flat[flat != 0]:
            hit[idx[float(v)]] += 1
        assert np.all(hit == 1)


def test_m_pad_closed_form(orc):
    for m, want in ((0, 0), (1, 16), (16, 16), (17, 32), (25, 32), (1168, 1168), (4576, 4576),
                    (16383, 16384)):
        assert orc.m_pad(m) == want


def test_weight_block_quant(orc):
    rng = np.random.default_rng(3)
    N, K = 256, 384
    w = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    q, s = orc.quant_weight_block(w)
    blocks = np.abs(w).reshape(N // 128, 128, K // 128, 128).max(axis=(1, 3))
    assert np.array_equal(s.view(np.uint32), (blocks / np.float32(448)).astype(np.float32).view(np.uint32))
    # each block's amax element(s) encode to +-448, and codes match numpy
    # division + torch cast
    sb = np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)
    qq = np.clip(w / sb, -448, 448).astype(np.float32)
    want = torch.from_numpy(qq).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, want)


def _lib_quant_codes(x_bits: np.ndarray) -> np.ndarray:
    """Reference codes from numpy IEEE fp32 division + torch's e4m3fn cast."""
    xf = bf16_bits_to_f32(x_bits)
    amax = np.abs(xf).max(axis=1, keepdims=True)
    s = (amax / np.float32(448.0)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        qv = np.where(s > 0, xf / np.where(s > 0, s, np.float32(1)), xf).astype(np.float32)
    qv = np.clip(qv, -448.0, 448.0).astype(np.float32)
    return torch.from_numpy(qv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.slow
def test_exhaustive_element_map(orc):
    """Every (x, amax) pair of finite bf16 values with |x| <= amax."""
    total = 0
    for lo, hi in synth.exhaustive_chunks(1 << 20):
        g = synth.exhaustive_pair_groups(lo, hi)
        q, s = orc.quant_act(g.reshape(1, -1))
        want = _lib_quant_codes(g)
        got = q.reshape(g.shape)
        if not np.array_equal(got, want):
            bad = np.argwhere(got != want)[:5]
            pytest.fail(f"amax chunk {lo:#x}..{hi:#x}: first mismatches at {bad.tolist()}")
        total += g.shape[0]
    assert total == synth.n_exhaustive_groups()
