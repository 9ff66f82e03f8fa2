"""Pins of the oracle's weight-format functions: per-row FP8 weights, the
FP8 -> bf16 weight dequantizer, and the GEMM reference under both weight
scale geometries.

Page "dispatch_proj.rs", doc of dequant_fp8_bf16_into: one index formula,
scale[(n/block_n)*sk + k/block_k], serves the 128x128 block-scaled format
(128, 128, K/128) and the per-row format (1, K, 1); an FP8 e4m3 value is
exact in bf16, so dequantization with a power-of-two scale loses nothing.

* per-row weight quantizer: scale = row amax / 448 and the codes of an
  independent brute-force encoder;
* dequantizer: bit-exact against torch's own float8 decode, float32 multiply
  and bf16 cast; exact (lossless) for power-of-two scales; both geometries
  address the scale the formula says, ragged N included;
* GEMM with per-row scales: numpy float64 matmul of the dequantized
  operands, and bit-equal to the block-scaled reference when the per-row
  scales are constant over each 128-row block.
"""
import numpy as np
import pytest
import torch

import brute
import synth


def _codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x00  # no NaN codes
    return c


def _torch_dequant(codes, scale_full):
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
    return (dec * torch.from_numpy(scale_full.astype(np.float32))).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def test_quant_weight_row_scales_and_codes(orc):
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.02, (7, 384)).astype(np.float32)
    w[3] = 0.0                     # all-zero row: scale 0, signed-zero codes
    w[4, 10] = 3.0                 # one outlier
    q, s = orc.quant_weight_row(w)
    amax = np.abs(w).max(axis=1).astype(np.float32)
    assert np.array_equal(s, (amax / np.float32(448.0)).astype(np.float32))
    for n in (0, 3, 4, 6):
        for k in range(0, 384, 37):
            x = float(w[n, k])
            want = (0x80 if np.signbit(w[n, k]) else 0) if s[n] == 0 else brute.encode(
                brute.f32(x / float(s[n])))
            assert q[n, k] == want, (n, k)
    assert q[4, 10] == 0x7E  # the row maximum maps to 448


@pytest.mark.parametrize("N,K", [(128, 256), (300, 384), (5, 1280)])
def test_dequant_matches_torch_both_geometries(orc, N, K):
    rng = np.random.default_rng(N * 3 + K)
    codes = _codes(rng, (N, K))
    # per-row
    s_row = (rng.random(N) * 0.01 + 1e-4).astype(np.float32)
    got = orc.dequant_fp8_bf16(codes, s_row)
    assert np.array_equal(got, _torch_dequant(codes, np.repeat(s_row[:, None], K, axis=1)))
    # 128x128 blocks (ceil(N/128) scale rows)
    nb = (N + 127) // 128
    s_blk = (rng.random((nb, K // 128)) * 0.01 + 1e-4).astype(np.float32)
    full = np.repeat(np.repeat(s_blk, 128, axis=0), 128, axis=1)[:N]
    got = orc.dequant_fp8_bf16(codes, s_blk)
    assert np.array_equal(got, _torch_dequant(codes, full))


def test_dequant_power_of_two_scales_are_lossless(orc):
    rng = np.random.default_rng(9)
    codes = _codes(rng, (256, 256))
    s_blk = np.ldexp(1.0, rng.integers(-20, 6, (2, 2))).astype(np.float32)
    got = synth.bf16_bits_to_f32(orc.dequant_fp8_bf16(codes, s_blk)).astype(np.float64)
    exact = orc.e4m3_decode(codes) * np.repeat(np.repeat(s_blk.astype(np.float64), 128, 0), 128, 1)
    assert np.array_equal(got, exact)


def test_dequant_scale_index(orc):
    """Each element takes the scale the index formula names: isolate scales
    with codes 0x38 (= 1.0) and distinct powers of two."""
    N, K = 260, 384
    codes = np.full((N, K), 0x38, dtype=np.uint8)
    s_blk = np.ldexp(1.0, np.arange(9).reshape(3, 3) - 4).astype(np.float32)
    v = synth.bf16_bits_to_f32(orc.dequant_fp8_bf16(codes, s_blk))
    for n in (0, 127, 128, 255, 256, 259):
        for k in (0, 127, 128, 383):
            assert v[n, k] == s_blk[n // 128, k // 128], (n, k)
    s_row = np.ldexp(1.0, (np.arange(N) % 17) - 8).astype(np.float32)
    v = synth.bf16_bits_to_f32(orc.dequant_fp8_bf16(codes, s_row))
    assert np.array_equal(v, np.repeat(s_row[:, None], K, axis=1))


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (16, 200, 512), (37, 384, 640)])
def test_gemm_rowscale_matches_numpy_dgemm(orc, M, N, K):
    rng = np.random.default_rng(M + N + K + 1)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a, a_s = orc.quant_act(x)
    w, w_s = orc.quant_weight_row(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    ref = orc.gemm_ref(a, a_s, w, w_s)
    A = orc.e4m3_decode(a) * np.repeat(a_s.astype(np.float64), 128, axis=1)
    Wd = orc.e4m3_decode(w) * w_s.astype(np.float64)[:, None]
    want = A @ Wd.T
    assert np.max(np.abs(ref - want)) <= 1e-12 * np.max(np.abs(want))
    ms = rng.integers(0, M, 50)
    ns = rng.integers(0, N, 50)
    assert np.array_equal(orc.gemm_ref_at(a, a_s, w, w_s, ms, ns), ref[ms, ns])


def test_gemm_rowscale_equals_block_when_constant_per_block(orc):
    M, N, K = 9, 256, 384
    rng = np.random.default_rng(4)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a, a_s = orc.quant_act(x)
    w = _codes(rng, (N, K))
    s_blocks = (rng.random(N // 128) + 0.5).astype(np.float32)
    s_row = np.repeat(s_blocks, 128)
    s_blk = np.repeat(s_blocks[:, None], K // 128, axis=1)
    assert np.array_equal(orc.gemm_ref(a, a_s, w, s_row), orc.gemm_ref(a, a_s, w, s_blk))


def test_gemm_bf16_ref_integer_exact(orc):
    """Small-integer bf16 operands: the reference equals exact integer
    arithmetic."""
    rng = np.random.default_rng(12)
    xi = rng.integers(-8, 9, (7, 192))
    wi = rng.integers(-8, 9, (130, 192))
    xb = synth.f32_to_bf16_bits(xi.astype(np.float32))
    wb = synth.f32_to_bf16_bits(wi.astype(np.float32))
    assert np.array_equal(orc.gemm_bf16_ref(xb, wb), (xi @ wi.T).astype(np.float64))
