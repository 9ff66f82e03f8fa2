"""GPU parity of the dense FFN chain (page "dispatch_proj.rs", doc of
cublas_fp8_proj_prequant: the gate and up projections share one quantized
input; the post-SiLU intermediate is quantized once for down).

* fp8q_silu_mul_quant: the intermediate's codes and K-major scales against
  the oracle (silu_mul, quant_act, scale_to_kmajor), bit-exact in every group
  the oracle does not mark as holding an element a binary32 evaluation may
  round either way; such groups must equal the quantization of one of the
  intermediates the marks allow.  Ragged M, pad slots zero, canaries;
  deep-negative gates, zeros, signed zeros.
* fp8q_ffn_gate_up on exact special cases (small-integer codes, power-of-two
  scales: gate and up are exact in fp32) to the same bar, and bit-identical
  to the separate path (two GEMMs + fp8q_silu_mul_quant) on random data.
* fp8q_ffn end to end, both variants bit-identical to each other:
  - exact gate/up values (integer activations with power-of-two group
    scales, small-integer weights): the intermediate bit-exact modulo the
    SiLU's marked roundings and the output within the projection tolerance
    (relative RMS <= 1e-3 against the bf16-rounded reference, every element
    within one bf16 ulp + 1e-3 RMS), up to the full FFN width;
  - random data: the intermediate's codes differ from the oracle's only in
    a small fraction of positions, by about one step (the FP8 MFMA's
    accumulation error moves gate/up values across rounding boundaries),
    and the output
    is within the projection tolerance plus the derived effect of those
    codes; full FFN sizes (H=5120, I=17408) at decode, prefill (M=1168) and
    large prefill (M=4576) widths on one row of every 128-row tile.
"""
import dataclasses
import itertools

import numpy as np
import pytest
import torch

import synth
from gpu_util import Guarded, bf16_bits_to_f64, dev, host, log, require_gpu

pytestmark = pytest.mark.gpu

fp8q = None
RTOL = 1e-3
SKINNY_MAX_M = 64  # fp8q_gemm_blockscaled's automatic choice uses the skinny kernel up to here


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global fp8q
    require_gpu()
    import w8a8_fp8_block_amd as m
    fp8q = m
    yield


# ------------------------------------------------------------------ helpers
def _bf(vals):
    return synth.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def _neighbour(bits: int, d: int) -> int:
    """bf16 pattern one step up (d=1) or down (d=-1) in magnitude."""
    mag, sign = bits & 0x7FFF, bits & 0x8000
    if d == 0:
        return bits
    if d > 0:
        return sign | min(mag + 1, 0x7F7F)
    return sign | (mag - 1) if mag > 0 else (sign ^ 0x8000) | 1


def _km_to_rm(km, M):
    return np.ascontiguousarray(km[:, :M].T)


def _check_h_quant(orc, h, amb, codes_gpu, km_gpu, M, I):
    """GPU codes [M,I] and K-major scales [G, Mp] against the oracle's
    quantization of h = silu_mul(g, u); groups that differ must hold
    ambiguous elements and equal the quantization of an allowed h.
    Returns the number of groups resolved that way."""
    G, Mp = I // 128, synth.ceil16(M)
    assert km_gpu.shape == (G, Mp)
    assert np.all(km_gpu[:, M:].view(np.uint32) == 0), "pad slots must be +0"
    q, s = orc.quant_act(h)
    s_gpu = _km_to_rm(km_gpu, M)
    bad = (codes_gpu != q).reshape(M, G, 128).any(-1) | (s_gpu.view(np.uint32) != s.view(np.uint32))
    resolved = 0
    for m, gi in zip(*np.nonzero(bad)):
        sl = slice(128 * gi, 128 * gi + 128)
        idx = np.nonzero(amb[m, sl])[0]
        assert 0 < len(idx) <= 6, f"row {m} group {gi}: differs with {len(idx)} ambiguous elements"
        base = h[m, sl].copy()
        found = False
        for combo in itertools.product((0, 1, -1), repeat=len(idx)):
            cand = base.copy()
            for j, d in zip(idx, combo):
                cand[j] = _neighbour(int(cand[j]), d)
            cq, cs = orc.quant_act(cand[None, :])
            if np.array_equal(cq[0], codes_gpu[m, sl]) and \
                    cs.view(np.uint32)[0, 0] == s_gpu.view(np.uint32)[m, gi]:
                found = True
                break
        assert found, f"row {m} group {gi}: no allowed rounding of h gives the GPU result"
        resolved += 1
    return resolved


def _silu_mul_quant_gpu(g, u):
    M, I = g.shape
    hq = Guarded((M, I), torch.uint8)
    km = Guarded((I // 128, synth.ceil16(M)), torch.float32)
    fp8q.fp8q_silu_mul_quant(dev(g), dev(u), hq.t, km.t)
    torch.cuda.synchronize()
    hq.check_canary()
    km.check_canary()
    return host(hq.t), host(km.t)


def _gate_up_fused_gpu(xq, xs_km, gq, gs, uq, us):
    M, H = xq.shape
    I = gq.shape[0]
    hq = Guarded((M, I), torch.uint8)
    km = Guarded((I // 128, synth.ceil16(M)), torch.float32)
    fp8q.fp8q_ffn_gate_up(dev(xq), dev(xs_km), dev(gq), dev(gs), dev(uq), dev(us), hq.t, km.t)
    torch.cuda.synchronize()
    hq.check_canary()
    km.check_canary()
    return host(hq.t), host(km.t)


def _gate_up_separate_gpu(xq, xs_km, gq, gs, uq, us):
    M, H = xq.shape
    I = gq.shape[0]
    g = torch.empty((M, I), dtype=torch.int16, device="cuda")
    u = torch.empty((M, I), dtype=torch.int16, device="cuda")
    x_d, km_d = dev(xq), dev(xs_km)
    fp8q.fp8q_gemm_blockscaled(x_d, km_d, dev(gq), dev(gs), g)
    fp8q.fp8q_gemm_blockscaled(x_d, km_d, dev(uq), dev(us), u)
    hq = torch.empty((M, I), dtype=torch.uint8, device="cuda")
    km = torch.empty((I // 128, synth.ceil16(M)), dtype=torch.float32, device="cuda")
    fp8q.fp8q_silu_mul_quant(g, u, hq, km)
    torch.cuda.synchronize()
    return host(hq), host(km)


def _weights(orc, wf):
    return tuple(orc.quant_weight_block(a) for a in wf)


# ------------------------------------------------------ silu_mul_quant alone
@pytest.mark.parametrize("M,I", [(1, 128), (16, 384), (37, 1024), (300, 640), (1029, 256)])
def test_silu_mul_quant_matches_oracle(orc, M, I):
    rng = np.random.default_rng(M * 31 + I)
    g = _bf(rng.normal(0.0, 3.0, (M, I)))
    u = _bf(rng.normal(0.0, 2.0, (M, I)))
    # edge values in the first rows: deep negative gates, exact zeros, signed
    # zeros, large positive gates, up of zero
    e = min(M, 4)
    g[:e, :64] = _bf(np.linspace(-120.0, -60.0, 64))
    g[:e, 64:70] = _bf([0.0, -0.0, 0.0, -0.0, 200.0, -200.0])
    u[:e, 64:70] = _bf([1.0, 1.0, -1.0, -1.0, -3.0, 5.0])
    g[:e, 74:78] = _bf([3.0e38, -3.0e38, 1.0e30, -1.0e30])  # huge gates, finite products
    u[:e, 74:78] = _bf([1.0, 1.0, 1.0e-30, 1.0e-30])
    u[:e, 70:74] = _bf([0.0, -0.0, 0.0, -0.0])
    h, amb = orc.silu_mul(g, u)
    log(f"silu_mul_quant M={M} I={I}: {int(amb.sum())} ambiguous elements")
    codes, km = _silu_mul_quant_gpu(g, u)
    n = _check_h_quant(orc, h, amb, codes, km, M, I)
    log(f"  groups resolved through the ambiguity marks: {n}")


def test_silu_mul_quant_zero_groups_and_all_tail_group(orc):
    M, I = 3, 384
    g = _bf(np.full((M, I), 1.5))
    u = _bf(np.full((M, I), 2.0))
    u[0, :128] = _bf(np.zeros(128))          # a zero group: scale 0, codes +-0
    u[1, 128:256] = _bf(-np.zeros(128))      # negative zeros times positive silu
    g[2, 256:] = _bf(np.linspace(-100.0, -70.0, 128))  # every |h| below 2^-96
    h, amb = orc.silu_mul(g, u)
    codes, km = _silu_mul_quant_gpu(g, u)
    _check_h_quant(orc, h, amb, codes, km, M, I)
    assert np.all(codes[0, :128] == 0x00) and np.all(codes[1, 128:256] == 0x80)
    assert km[0, 0] == 0.0 and km[1, 1] == 0.0


# ------------------------------------------------------- fused gate/up stage
def _int_operands(orc, rng, M, H, I):
    """Small-integer codes, power-of-two scales: every gate/up value is an
    exact fp32 (and bf16) number."""
    xq = orc.e4m3_encode(rng.integers(-3, 4, (M, H)).astype(np.float32))
    xs = np.exp2(rng.integers(-3, 0, (M, H // 128))).astype(np.float32)
    gq = orc.e4m3_encode(rng.integers(-2, 3, (I, H)).astype(np.float32))
    uq = orc.e4m3_encode(rng.integers(-2, 3, (I, H)).astype(np.float32))
    gs = np.exp2(rng.integers(-5, -2, (I // 128, H // 128))).astype(np.float32)
    us = np.exp2(rng.integers(-5, -2, (I // 128, H // 128))).astype(np.float32)
    return xq, xs, gq, gs, uq, us


@pytest.mark.parametrize("M,H,I", [(1, 128, 128), (37, 256, 384), (130, 384, 256),
                                   (300, 256, 512), (16, 5120, 1024)])
def test_ffn_gate_up_exact_special_cases(orc, M, H, I):
    rng = np.random.default_rng(M + H + I)
    xq, xs, gq, gs, uq, us = _int_operands(orc, rng, M, H, I)
    g64 = orc.gemm_ref(xq, xs, gq, gs)
    u64 = orc.gemm_ref(xq, xs, uq, us)
    assert np.array_equal(g64.astype(np.float32).astype(np.float64), g64)
    g, u = orc.f64_to_bf16(g64), orc.f64_to_bf16(u64)
    h, amb = orc.silu_mul(g, u)
    km = orc.scale_to_kmajor(xs)
    log(f"gate/up exact M={M} H={H} I={I}")
    codes, hkm = _gate_up_fused_gpu(xq, km, gq, gs, uq, us)
    n = _check_h_quant(orc, h, amb, codes, hkm, M, I)
    log(f"  fused: {n} groups resolved through the ambiguity marks")
    codes2, hkm2 = _gate_up_separate_gpu(xq, km, gq, gs, uq, us)
    assert np.array_equal(codes, codes2) and np.array_equal(hkm.view(np.uint32), hkm2.view(np.uint32))


@pytest.mark.parametrize("M,H,I", [(37, 512, 384), (300, 1024, 768), (1300, 640, 512)])
def test_ffn_gate_up_fused_equals_separate(orc, M, H, I):
    w = synth.FfnWorkload("t", M, H, I, max(1, H // 100), 20.0, seed=M + I)
    x, wf = synth.make_ffn_inputs(w)
    (gq, gs), (uq, us), _ = _weights(orc, wf)
    xq, xs = orc.quant_act(x)
    km = orc.scale_to_kmajor(xs)
    log(f"gate/up fused vs separate M={M} H={H} I={I}")
    a = _gate_up_fused_gpu(xq, km, gq, gs, uq, us)
    b = _gate_up_separate_gpu(xq, km, gq, gs, uq, us)
    assert np.array_equal(a[0], b[0]), "codes differ"
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32)), "scales differ"


# -------------------------------------------------------------- whole chain
def _ffn_gpu(x, W, variant, M, H, I):
    (gq, gs), (uq, us), (dq, ds) = W
    out = Guarded((M, H), torch.int16)
    ws = fp8q.alloc_ffn_workspace(M, H, I, variant)
    fp8q.fp8q_ffn(dev(x), dev(gq), dev(gs), dev(uq), dev(us), dev(dq), dev(ds), out.t, ws,
                  variant=variant)
    torch.cuda.synchronize()
    out.check_canary()
    # the workspace keeps the intermediate: codes and K-major scales
    a256 = lambda v: (v + 255) // 256 * 256  # noqa: E731
    Mp = synth.ceil16(M)
    off_hq = a256(M * H) + a256(M * (H // 128) * 4) + a256(Mp * (H // 128) * 4)
    off_hs = a256(off_hq + M * I)
    wsh = host(ws)
    hq = wsh[off_hq:off_hq + M * I].reshape(M, I)
    hs = wsh[off_hs:off_hs + Mp * (I // 128) * 4].view(np.float32).reshape(I // 128, Mp)
    return host(out.t).view(np.uint16), hq, hs


def _exact_ffn_inputs(rng, M, H, I):
    """Activations of small integers with a +-7 in every 128-group (scale
    7/448 = 2^-6, every code exact), weights of small-integer codes with
    power-of-two block scales: gate and up are exact in fp32 whatever the
    order of the sums, so the only rounding before the intermediate is the
    SiLU's."""
    xi = rng.integers(-7, 8, (M, H)).astype(np.float32)
    xi[:, ::128] = np.where(rng.random((M, H // 128)) < 0.5, -7.0, 7.0)
    x = synth.f32_to_bf16_bits(xi)
    W = []
    for n, k in ((I, H), (I, H), (H, I)):
        q = rng.integers(-2, 3, (n, k)).astype(np.float32)
        s = np.exp2(rng.integers(-7, -4, (n // 128, k // 128))).astype(np.float32)
        W.append((q, s))
    return x, W


@pytest.mark.parametrize("M,H,I,rows", [(1, 1024, 1536, None), (37, 1024, 1536, None),
                                        (200, 1024, 1536, None), (16, 5120, 17408, None),
                                        (300, 5120, 17408, 5)])
def test_ffn_exact_gate_up_chain(orc, M, H, I, rows):
    """Whole chain with exact gate/up values: the intermediate bit-exact
    (modulo the SiLU's marked roundings), the output within the projection
    tolerance of the oracle (the down GEMM is the only inexact step)."""
    rng = np.random.default_rng(M + H + I)
    x, Wf = _exact_ffn_inputs(rng, M, H, I)
    W = tuple((orc.e4m3_encode(q), s) for q, s in Wf)
    sel = np.arange(M) if rows is None else np.unique(
        np.concatenate([[0, M - 1], rng.integers(0, M, rows)]))
    ref = orc.ffn_ref(x, *W[0], *W[1], *W[2], rows=sel)
    assert np.array_equal(orc.e4m3_decode(ref["xq"]) * np.repeat(ref["xs"], 128, axis=1),
                          synth.bf16_bits_to_f32(x[sel]).astype(np.float64))
    outs = {}
    for variant in (1, 2):
        log(f"ffn exact M={M} H={H} I={I} variant={variant}")
        out, hq, hs = _ffn_gpu(x, W, variant, M, H, I)
        outs[variant] = (out, hq)
        hq_s, hs_s = hq[sel], np.ascontiguousarray(hs[:, sel])
        hs_s = np.concatenate([hs_s, np.zeros((hs.shape[0], synth.ceil16(len(sel)) - len(sel)),
                                              np.float32)], axis=1)
        assert np.all(hs[:, M:].view(np.uint32) == 0), "pad slots must be +0"
        n = _check_h_quant(orc, ref["h"], ref["amb"], hq_s, hs_s, len(sel), I)
        log(f"  intermediate bit-exact ({n} groups resolved through the SiLU marks)")
        # reference output from the intermediate the GPU holds, which the
        # check above has shown to be one of the allowed ones
        r = orc.gemm_ref(hq_s, _km_to_rm(hs_s, len(sel)), *W[2]) if n else ref["out"]
        rel, exc, relf = orc.gemm_errors(bf16_bits_to_f64(out[sel]), r)
        log(f"  out: rel_rms={rel:.3e} (vs fp64 {relf:.3e}) worst/bound={exc:.3f}")
        assert rel <= RTOL and exc <= 1.0
    assert np.array_equal(outs[1][0], outs[2][0]) and np.array_equal(outs[1][1], outs[2][1])


def _check_random_chain(orc, ref, out_bits, hq, hs, rows, what):
    """Random data: gate and up carry the FP8 MFMA's accumulation error (the
    128-product dot product of one instruction is formed to about 2^-15 of
    its largest product, not to fp32 rounding), so near a bf16 or e4m3
    rounding boundary the GPU's intermediate can take the other code.
    Checks: at most 3% of the intermediate's codes differ from the oracle's,
    each dequantized value within one e4m3 step plus 2^-5 of the group
    maximum of the oracle's; at most 3% of the group scales (or 2, for few
    groups) differ, each within 2^-5; the output's relative
    RMS error is within the projection's 1e-3 plus the effect of the
    differing codes, at most 0.25 * sqrt(f) for a fraction f of terms each
    moved by one e4m3 step (at most 1/8 of its value)."""
    M = hq.shape[0]
    cq, rq = hq[rows], ref["hq"]
    diff = cq != rq
    s_gpu = _km_to_rm(hs, M)[rows]
    sdiff = s_gpu.view(np.uint32) != ref["hs"].view(np.uint32)
    f = float(diff.mean())
    log(f"  {what}: intermediate codes differing {int(diff.sum())}/{diff.size} (f={f:.2e}), "
        f"scales differing {int(sdiff.sum())}/{sdiff.size}")
    assert f <= 0.03 and sdiff.sum() <= max(2, 0.03 * sdiff.size)
    if sdiff.any():
        r = s_gpu[sdiff] / ref["hs"][sdiff]
        log(f"  {what}: differing scales within {float(np.max(np.abs(r - 1.0))):.2e} relative")
        assert np.all(np.abs(r - 1.0) <= 2.0 ** -5), r
    # each differing element: the two dequantized values within one e4m3
    # step (at the larger of the two) plus 2^-5 of the group maximum (the
    # gate/up error, up to 2^-12 of the largest product of each block --
    # outlier channels make that large next to small outputs -- carried
    # through silu * up)
    s_g = np.repeat(s_gpu, 128, axis=1).astype(np.float64)
    s_o = np.repeat(ref["hs"], 128, axis=1).astype(np.float64)
    vg = orc.e4m3_decode(cq) * s_g
    vo = orc.e4m3_decode(rq) * s_o
    big = np.maximum(np.abs(vg) / s_o, np.abs(vo) / s_o)  # in units of the oracle's scale
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(big > 0, big, 1.0)))
    step = np.where(big >= 2.0 ** -6, np.exp2(e - 3), 2.0 ** -9) * s_o
    slack = step + 2.0 ** -5 * 448.0 * s_o
    worst = float(np.max((np.abs(vg - vo) / slack)[diff])) if diff.any() else 0.0
    log(f"  {what}: worst differing element / (one step + 2^-5 amax) = {worst:.3f}")
    assert worst <= 1.0
    o = bf16_bits_to_f64(out_bits[rows])
    rel, exc, relf = orc.gemm_errors(o, ref["out"])
    bound = RTOL + 0.25 * np.sqrt(f)
    log(f"  {what}: out rel_rms={rel:.3e} (bound {bound:.3e}), worst/bound={exc:.3f}")
    assert rel <= bound


@pytest.mark.parametrize("M", [1, 16, 25, 200])
def test_ffn_random_small_widths(orc, M):
    w = synth.FfnWorkload("t", M, 1024, 1536, 10, 20.0, seed=M)
    x, wf = synth.make_ffn_inputs(w)
    W = _weights(orc, wf)
    ref = orc.ffn_ref(x, *W[0], *W[1], *W[2])
    rows = np.arange(M)
    outs = {}
    for variant in (1, 2, 0):
        log(f"ffn M={M} H=1024 I=1536 variant={variant}")
        outs[variant] = _ffn_gpu(x, W, variant, M, 1024, 1536)
        _check_random_chain(orc, ref, *outs[variant], rows, f"variant {variant}")
    auto = fp8q.fp8q_ffn_select(M, 1024, 1536)
    assert np.array_equal(outs[0][0], outs[auto][0])
    if M > SKINNY_MAX_M:  # both variants' gate/up sums run in the same order
        assert np.array_equal(outs[1][0], outs[2][0]) and np.array_equal(outs[1][1], outs[2][1])


@pytest.mark.parametrize("name,M", [("ffn_decode", 16), ("ffn_decode", 25), ("ffn_prefill", 256),
                                    ("ffn_prefill", 1168), ("ffn_large", 4576)])
def test_ffn_full_size_sampled_rows(orc, name, M):
    """Full model widths, checked on one row of every 128-row tile (every row
    at decode widths); M = 256 at the prefill widths is a row count whose
    down projection runs split-K."""
    base = synth.ffn_workload(name)
    w = synth.ffn_workload(name, M) if M in [v.M for v in synth.FFN_WORKLOADS[name]] else \
        dataclasses.replace(base, M=M)
    log(f"ffn {w.desc}: drawing inputs")
    x, wf = synth.make_ffn_inputs(w)
    W = _weights(orc, wf)
    del wf
    rng = np.random.default_rng(M)
    # the first and last rows and one random row of every 128-row tile
    # (all rows at decode widths)
    per_tile = [rng.integers(m0, min(m0 + 128, M), 1) for m0 in range(0, M, 128)]
    rows = np.arange(M) if M <= 64 else np.unique(np.concatenate([[0, M - 1], *per_tile]))
    log(f"  oracle on rows {rows.tolist()}")
    ref = orc.ffn_ref(x, *W[0], *W[1], *W[2], rows=rows)
    log(f"  fp8q_ffn variant {fp8q.fp8q_ffn_select(M, w.H, w.I)}")
    out, hq, hs = _ffn_gpu(x, W, 0, M, w.H, w.I)
    _check_random_chain(orc, ref, out, hq, hs, rows, f"{w.desc} auto")
    other = 2 if fp8q.fp8q_ffn_select(M, w.H, w.I) == 1 else 1
    log(f"  fp8q_ffn variant {other}")
    out2, hq2, hs2 = _ffn_gpu(x, W, other, M, w.H, w.I)
    if M > SKINNY_MAX_M:
        assert np.array_equal(out, out2) and np.array_equal(hq, hq2)
    else:  # the skinny GEMMs split K over waves: another summation order
        _check_random_chain(orc, ref, out2, hq2, hs2, rows, f"{w.desc} variant {other}")
