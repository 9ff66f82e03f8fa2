"""GPU parity of the block-scaled FP8 GEMM and of the whole projection.

Accuracy contract against the oracle's fp64 block-form product r:
  rel_rms = sqrt(sum (o-b)^2 / sum b^2) <= 1e-3 with b = r rounded to bf16
  (the output format; rounding alone puts any bf16 output ~1.66e-3 away from
  the unrounded r), and for every element |o - r| <= ulp_bf16(r) + 1e-3*RMS(r).
The whole output is compared at every size, the full prefill projections
(M=1168, N=17408, K=5120 and M=4576, N=5120, K=17408) included: every kernel
the API can force, the split-K form, and the whole projection (fp8q_proj)
against the oracle's full fp64 product; the tiled kernels' outputs must be
bit-identical to each other and to a repeated launch of themselves.  Exact
special cases (powers of two, one-hot rows, small integers) must match bit
for bit, and a wrong scale layout must fail by a wide margin.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import RTOL, Guarded, bf16_bits_to_f64, dev, host, log, require_gpu, assert_tol

pytestmark = pytest.mark.gpu

fp8q = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global fp8q
    require_gpu()
    import w8a8_fp8_block_amd as m
    fp8q = m
    yield


def _operands(orc, w: synth.Workload, M=None):
    x, wf, _ = synth.make_inputs(w, M=M)
    a, a_s = orc.quant_act(x)
    wq, ws = orc.quant_weight_block(wf)
    return x, a, a_s, wq, ws


def _gemm_gpu(orc, a, a_s, wq, ws, kernel=0, km=None):
    M, K = a.shape
    N = wq.shape[0]
    if km is None:
        km = orc.scale_to_kmajor(a_s)
    out = Guarded((M, N), torch.int16)
    fp8q.fp8q_gemm_blockscaled(dev(a), dev(km), dev(wq), dev(ws), out.t, kernel=kernel)
    torch.cuda.synchronize()
    out.check_canary()
    return bf16_bits_to_f64(host(out.t))


def orc_errors(o, r, rms=None):
    import oracle
    return oracle.gemm_errors(o, r, rms)


def _kernels_for(M, N=256):
    """Every kernel the API can force for this shape: auto, the default tiled
    kernel, the skinny kernel (row tiles of 64 beyond 64 rows) and the other
    tile shapes."""
    return (0, 1, 2, 3, 4, 5)


@pytest.mark.parametrize("M,N,K", [(16, 256, 512), (1, 128, 128), (17, 384, 640), (33, 256, 1152),
                                   (64, 128, 256), (130, 384, 640), (257, 256, 384),
                                   (300, 512, 896)])
def test_gemm_small_full(orc, M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a, a_s = orc.quant_act(x)
    wq, ws = orc.quant_weight_block(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    ref = orc.gemm_ref(a, a_s, wq, ws)
    for kern in _kernels_for(M, N):
        log(f"gemm M={M} N={N} K={K} kernel={kern}")
        assert_tol(_gemm_gpu(orc, a, a_s, wq, ws, kern), ref, f"M{M}N{N}K{K}k{kern}")


def test_gemm_tiny_workload(orc):
    w = synth.workload("tiny")
    _, a, a_s, wq, ws = _operands(orc, w)
    ref = orc.gemm_ref(a, a_s, wq, ws)
    for kern in _kernels_for(w.M, w.N):
        log(f"gemm tiny kernel={kern}")
        assert_tol(_gemm_gpu(orc, a, a_s, wq, ws, kern), ref, f"tiny k{kern}")


@pytest.mark.parametrize("M", [16, 17, 25])
def test_gemm_decode_workload_full(orc, M):
    w = synth.workload("decode", M=M)
    _, a, a_s, wq, ws = _operands(orc, w)
    log(f"oracle decode M={M}")
    ref = orc.gemm_ref(a, a_s, wq, ws)
    for kern in _kernels_for(M, w.N):
        log(f"gemm decode M={M} kernel={kern}")
        assert_tol(_gemm_gpu(orc, a, a_s, wq, ws, kern), ref, f"decode M{M} k{kern}")


_FULL = {}


def _full_size(orc, name):
    """Operands of a full-size projection workload on host and device and the
    oracle's fp64 product over all M*N outputs (one workload kept at a time)."""
    if name not in _FULL:
        _FULL.clear()
        w = synth.WORKLOADS[name][0]
        log(f"inputs {w.desc}")
        x, a, a_s, wq, ws = _operands(orc, w)
        log(f"oracle {w.desc}: full fp64 product")
        ref = orc.gemm_ref(a, a_s, wq, ws)
        d = {"w": w, "x": x, "a": a, "a_s": a_s, "wq": wq, "ws": ws, "ref": ref,
             "a_d": dev(a), "km_d": dev(orc.scale_to_kmajor(a_s)), "wq_d": dev(wq),
             "ws_d": dev(ws)}
        _FULL[name] = d
    return _FULL[name]


def _gemm_dev(d, kernel, canary=True):
    """fp8q_gemm_blockscaled on the resident operands of d; the raw bf16 bits."""
    M, N = d["w"].M, d["w"].N
    out = Guarded((M, N), torch.int16)
    fp8q.fp8q_gemm_blockscaled(d["a_d"], d["km_d"], d["wq_d"], d["ws_d"], out.t, kernel=kernel)
    torch.cuda.synchronize()
    if canary:
        out.check_canary()
    return host(out.t).view(np.uint16)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["prefill", "large_prefill"])
def test_gemm_full_size_every_kernel(orc, name):
    """Every forceable kernel at the full prefill sizes, all M*N outputs against
    the oracle; the tiled kernels (1, 3, 4, 5) and the automatic choice are
    bit-identical (they add the scaled block products in the same order)."""
    d = _full_size(orc, name)
    bits = {}
    for kern in (0, 1, 2, 3, 4, 5):
        log(f"gemm {d['w'].desc} kernel={kern}")
        o = _gemm_dev(d, kern)
        assert_tol(bf16_bits_to_f64(o), d["ref"], f"{d['w'].desc} k{kern}")
        if kern != 2:
            bits[kern] = o
    for kern in (0, 3, 4, 5):
        assert np.array_equal(bits[kern], bits[1]), f"kernel {kern} differs from kernel 1"


@pytest.mark.slow
@pytest.mark.parametrize("name", ["prefill", "large_prefill"])
def test_gemm_full_size_repeat_bit_identical(orc, name):
    """Race detector: four launches of the automatic kernel back to back (no
    host synchronization between them) into four outputs, two more of the
    128x128 kernel and three of the stream-K form (fp8q_gemm_blockscaled_
    streamk on one workgroup per CU, one workspace shared by the three), all
    M*N outputs compared bit for bit."""
    d = _full_size(orc, name)
    M, N = d["w"].M, d["w"].N
    for kern in (0, 1):
        outs = [Guarded((M, N), torch.int16) for _ in range(4 if kern == 0 else 2)]
        log(f"gemm {d['w'].desc} kernel={kern} x{len(outs)} back to back")
        for g in outs:
            fp8q.fp8q_gemm_blockscaled(d["a_d"], d["km_d"], d["wq_d"], d["ws_d"], g.t, kernel=kern)
        torch.cuda.synchronize()
        first = host(outs[0].t)
        for i, g in enumerate(outs):
            g.check_canary()
            assert np.array_equal(host(g.t), first), f"kernel {kern}: launch {i} differs"
    w = d["w"]
    need = fp8q.fp8q_gemm_streamk_workspace_bytes(0)
    work = torch.empty((need // 4,), dtype=torch.float32, device="cuda")
    outs = [Guarded((M, N), torch.int16) for _ in range(3)]
    log(f"gemm {w.desc} stream-K x3 back to back")
    for g in outs:
        fp8q.fp8q_gemm_blockscaled_streamk(d["a_d"], d["km_d"], d["wq_d"], d["ws_d"], g.t, work)
    torch.cuda.synchronize()
    first = host(outs[0].t)
    for i, g in enumerate(outs):
        g.check_canary()
        assert np.array_equal(host(g.t), first), f"stream-K: launch {i} differs"


@pytest.mark.slow
@pytest.mark.parametrize("name", ["prefill", "large_prefill"])
def test_gemm_splitk_full_size(orc, name):
    """The workspace forms at the full prefill sizes (the automatic choice,
    the single-pass kernel at both; split-K at two forced counts; the
    stream-K form on one workgroup per CU: 720 and 680 tiles, two whole
    rounds and a tail of 208 and 168 tiles cut in two pieces along K), all
    M*N outputs against the oracle, workspace canaries checked."""
    d = _full_size(orc, name)
    w = d["w"]
    M, N, K = w.M, w.N, w.K
    for splits in (0, 2, 3):
        need = fp8q.fp8q_gemm_splitk_workspace_bytes(M, N, K, splits)
        log(f"splitk {w.desc} splits={splits} workspace={need}")
        out = Guarded((M, N), torch.int16)
        work = Guarded((max(need, 16) // 4,), torch.float32, fill=0x7F) if need else None
        fp8q.fp8q_gemm_blockscaled_splitk(d["a_d"], d["km_d"], d["wq_d"], d["ws_d"], out.t,
                                          None if work is None else work.t, splits=splits)
        torch.cuda.synchronize()
        out.check_canary()
        if work is not None:
            work.check_canary()
        assert_tol(bf16_bits_to_f64(host(out.t)), d["ref"], f"{w.desc} splitk s{splits}")
    need = fp8q.fp8q_gemm_streamk_workspace_bytes(0)
    log(f"streamk {w.desc} workspace={need}")
    out = Guarded((M, N), torch.int16)
    work = Guarded((need // 4,), torch.float32, fill=0x7F)
    fp8q.fp8q_gemm_blockscaled_streamk(d["a_d"], d["km_d"], d["wq_d"], d["ws_d"], out.t, work.t)
    torch.cuda.synchronize()
    out.check_canary()
    work.check_canary()
    assert_tol(bf16_bits_to_f64(host(out.t)), d["ref"], f"{w.desc} streamk")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["prefill", "large_prefill"])
def test_proj_full_size(orc, name):
    """fp8q_proj end to end at the full prefill sizes (M=1168: one kernel
    writes both scale layouts; M=4576: the quantizer and the relayout run
    separately): codes and both scale layouts bit-exact, all M*N outputs
    within the tolerance of the oracle."""
    d = _full_size(orc, name)
    w = d["w"]
    M, N, K = w.M, w.N, w.K
    assert fp8q.fp8q_proj_quant_fused(M, K) == (name == "prefill")
    out = Guarded((M, N), torch.int16)
    aq = Guarded((M, K), torch.uint8)
    asr = Guarded((M, K // 128), torch.float32)
    askm = Guarded((K // 128, synth.ceil16(M)), torch.float32, fill=0x7F)
    log(f"proj {w.desc}")
    fp8q.fp8q_proj(dev(d["x"]), d["wq_d"], d["ws_d"], out.t, aq.t, asr.t, askm.t)
    torch.cuda.synchronize()
    for g in (out, aq, asr, askm):
        g.check_canary()
    assert np.array_equal(host(aq.t), d["a"])
    assert np.array_equal(host(asr.t).view(np.uint32), d["a_s"].view(np.uint32))
    assert np.array_equal(host(askm.t).view(np.uint32),
                          orc.scale_to_kmajor(d["a_s"]).view(np.uint32))
    assert_tol(bf16_bits_to_f64(host(out.t)), d["ref"], f"proj {w.desc}")


def test_full_size_release():
    _FULL.clear()


def test_gemm_block_scale_isolation_exact(orc):
    """All codes 1.0, a_s[m,g] = 2^(m%5), w_s[nb,g] = 2^g * (nb+1): the result
    128 * (nb+1) * sum_g 2^(m%5+g) is exact in fp32 and in bf16."""
    M, N, K = 40, 384, 512
    G = K // 128
    a = np.full((M, K), 0x38, dtype=np.uint8)
    wq = np.full((N, K), 0x38, dtype=np.uint8)
    a_s = np.array([[2.0 ** (m % 5)] * G for m in range(M)], dtype=np.float32)
    ws = np.array([[2.0 ** g * (nb + 1) for g in range(G)] for nb in range(N // 128)], dtype=np.float32)
    ref = orc.gemm_ref(a, a_s, wq, ws)
    for kern in _kernels_for(M, N):
        o = _gemm_gpu(orc, a, a_s, wq, ws, kern)
        assert np.array_equal(o, ref), f"kernel {kern}"


def test_gemm_one_hot_rows_exact(orc):
    M, N, K = 48, 256, 640
    G = K // 128
    rng = np.random.default_rng(2)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a, _ = orc.quant_act(x)
    a_s = np.exp2(rng.integers(-6, 6, (M, G))).astype(np.float32)  # exact products
    kk = rng.integers(0, K, size=N)
    wq = np.zeros((N, K), dtype=np.uint8)
    wq[np.arange(N), kk] = 0x38
    ws = np.exp2(rng.integers(-3, 4, (N // 128, G))).astype(np.float32)
    ref = orc.gemm_ref(a, a_s, wq, ws)
    want = bf16_bits_to_f64(synth.f32_to_bf16_bits(ref.astype(np.float32)))  # exact in fp32
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    for kern in _kernels_for(M, N):
        o = _gemm_gpu(orc, a, a_s, wq, ws, kern)
        assert np.array_equal(o, want), f"kernel {kern}"


def test_gemm_small_integers_exact(orc):
    """Codes of small integers and power-of-two scales: every partial sum is an
    exact fp32 integer, so the GPU result must equal the bf16 rounding of the
    exact value."""
    M, N, K = 37, 256, 768
    G = K // 128
    rng = np.random.default_rng(4)
    ints = rng.integers(-3, 4, (M, K)).astype(np.float32)
    intw = rng.integers(-3, 4, (N, K)).astype(np.float32)
    a = orc.e4m3_encode(ints)
    wq = orc.e4m3_encode(intw)
    a_s = np.exp2(rng.integers(-2, 3, (M, G))).astype(np.float32)
    ws = np.exp2(rng.integers(-2, 3, (N // 128, G))).astype(np.float32)
    ref = orc.gemm_ref(a, a_s, wq, ws)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    want = bf16_bits_to_f64(synth.f32_to_bf16_bits(ref.astype(np.float32)))
    for kern in _kernels_for(M, N):
        o = _gemm_gpu(orc, a, a_s, wq, ws, kern)
        assert np.array_equal(o, want), f"kernel {kern}"


def test_gemm_rowmajor_scales_fail(orc):
    """Negative control: the quantizer's row-major scales handed over as if they
    were K-major (the measurement-control reading on the page
    "dispatch_proj.rs", cublas_scale_layout_kmajor) must miss the tolerance by
    far more than 10x."""
    M, N, K = 32, 256, 2048
    rng = np.random.default_rng(8)
    x = synth.f32_to_bf16_bits((rng.standard_normal((M, K)) *
                                np.exp(rng.uniform(-2, 2, (M, 1)))).astype(np.float32))
    a, a_s = orc.quant_act(x)
    wq, ws = orc.quant_weight_block(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    ref = orc.gemm_ref(a, a_s, wq, ws)
    Mp = synth.ceil16(M)
    wrong = np.zeros((K // 128) * Mp, dtype=np.float32)
    wrong[: a_s.size] = a_s.ravel()
    wrong = wrong.reshape(K // 128, Mp)
    for kern in _kernels_for(M, N):
        o = _gemm_gpu(orc, a, a_s, wq, ws, kern, km=wrong)
        rel, exc, _ = orc_errors(o, ref)
        log(f"  row-major control kernel {kern}: rel_rms={rel:.3e} worst/bound={exc:.1f}")
        assert rel > 10 * RTOL and exc > 10


# a shape past the fused-quantizer limit (3900 * 17408/128 = 530400 scale
# groups > 2^19), so fp8q_proj runs the quantizer and the relayout separately
_PROJ_SPLIT = synth.Workload("proj_split", 3900, 17408, 256, "laplace", 87, 50.0)


@pytest.mark.parametrize("name,M", [("tiny", None), ("decode", 16), ("decode", 17), ("decode", 25),
                                    ("prefill", 130), ("proj_split", None)])
def test_proj_end_to_end(orc, name, M):
    if name == "proj_split":
        w = _PROJ_SPLIT
    else:
        w = synth.workload(name) if M is None or name != "decode" else synth.workload(name, M=M)
    x, wf, _ = synth.make_inputs(w, M=M)
    assert fp8q.fp8q_proj_quant_fused(x.shape[0], w.K) == (name != "proj_split")
    Mr = x.shape[0]
    a, a_s = orc.quant_act(x)
    km_ref = orc.scale_to_kmajor(a_s)
    wq, ws = orc.quant_weight_block(wf)
    ref = orc.gemm_ref(a, a_s, wq, ws)
    log(f"proj {w.desc} M={Mr}")
    out = Guarded((Mr, w.N), torch.int16)
    aq = Guarded((Mr, w.K), torch.uint8)
    asr = Guarded((Mr, w.K // 128), torch.float32)
    askm = Guarded((w.K // 128, synth.ceil16(Mr)), torch.float32, fill=0x7F)
    fp8q.fp8q_proj(dev(x), dev(wq), dev(ws), out.t, aq.t, asr.t, askm.t)
    torch.cuda.synchronize()
    for g in (out, aq, asr, askm):
        g.check_canary()
    assert np.array_equal(host(aq.t), a)
    assert np.array_equal(host(asr.t).view(np.uint32), a_s.view(np.uint32))
    assert np.array_equal(host(askm.t).view(np.uint32), km_ref.view(np.uint32))
    assert_tol(bf16_bits_to_f64(host(out.t)), ref, f"proj {w.desc}")


def test_gemm_repeatable(orc):
    """Same inputs, same bits, run to run (no data races in the reduction)."""
    w = synth.workload("decode", M=25)
    _, a, a_s, wq, ws = _operands(orc, w)
    for kern in _kernels_for(25, w.N):
        o1 = _gemm_gpu(orc, a, a_s, wq, ws, kern)
        o2 = _gemm_gpu(orc, a, a_s, wq, ws, kern)
        assert np.array_equal(o1, o2)


def test_gemm_long_k_weight_scale_chunks(orc):
    """K spanning more than 1024 scale blocks, the weight scales of the later
    blocks clearly different from the earlier ones (a scale taken from the
    wrong K block shows)."""
    M, N, K = 40, 256, 1030 * 128
    rng = np.random.default_rng(21)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a, a_s = orc.quant_act(x)
    wq, ws = orc.quant_weight_block(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    # make the weight scales of the second chunk clearly different
    ws[:, 1024:] *= 3.0
    log(f"oracle M={M} N={N} K={K}")
    ref = orc.gemm_ref(a, a_s, wq, ws)
    for kern in _kernels_for(M, N):
        log(f"gemm long-K kernel={kern}")
        assert_tol(_gemm_gpu(orc, a, a_s, wq, ws, kern), ref, f"long-K k{kern}")


@pytest.mark.parametrize("M,N,K", [(300, 384, 1280), (1168, 512, 2048), (4576, 256, 640),
                                   (2300, 384, 256), (260, 384, 384), (300, 256, 768),
                                   (520, 384, 896), (300, 256, 1152), (260, 128, 128)])
def test_tiled_kernels_bit_identical(orc, M, N, K):
    """The tiled kernels (all tile shapes) add the scaled block products in the
    same order, so their outputs agree bit for bit; the auto choice is one of
    them.  The K loops are unrolled by the LDS stage count (3, or 6 where the
    register double buffer alternates too): K/128 here, 1, 2, 3, 5, 6, 7, 9,
    10 and 16, takes every residue mod 6, so each unrolled loop's tail length
    is exercised."""
    rng = np.random.default_rng(M + N + K)
    x = synth.f32_to_bf16_bits(rng.laplace(0, 1, (M, K)).astype(np.float32))
    a, a_s = orc.quant_act(x)
    wq, ws = orc.quant_weight_block(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    outs = {}
    for kern in (1, 3, 4, 5, 0):
        log(f"gemm M={M} N={N} K={K} kernel={kern}")
        outs[kern] = _gemm_gpu(orc, a, a_s, wq, ws, kern)
    for kern in (3, 4, 5, 0):
        assert np.array_equal(outs[kern], outs[1]), f"kernel {kern} differs from kernel 1"


@pytest.mark.parametrize("M,N,K", [(17, 384, 640), (25, 256, 1152), (130, 640, 896)])
def test_proj_deterministic_pattern(orc, M, N, K):
    """The whole projection on deterministic, seed-free data of the form
    ((k * 7919) mod 1013 - 506) / 97 over the flat element index (activations)
    and the same form scaled by 1/50 with an offset index (weights), at widths
    that are not tile multiples: codes and scales bit-exact, output within the
    projection tolerance of the oracle."""
    k = np.arange(M * K, dtype=np.int64)
    x = synth.f32_to_bf16_bits((((k * 7919) % 1013 - 506) / 97.0).astype(np.float32).reshape(M, K))
    kw = np.arange(N * K, dtype=np.int64) + 12345
    wf = ((((kw * 7919) % 1013 - 506) / 97.0) / 50.0).astype(np.float32).reshape(N, K)
    a, a_s = orc.quant_act(x)
    wq, ws = orc.quant_weight_block(wf)
    out = Guarded((M, N), torch.int16)
    aq = Guarded((M, K), torch.uint8)
    asr = Guarded((M, K // 128), torch.float32)
    askm = Guarded((K // 128, synth.ceil16(M)), torch.float32, fill=0x7F)
    fp8q.fp8q_proj(dev(x), dev(wq), dev(ws), out.t, aq.t, asr.t, askm.t)
    torch.cuda.synchronize()
    for g in (out, aq, asr, askm):
        g.check_canary()
    assert np.array_equal(host(aq.t), a)
    assert np.array_equal(host(asr.t).view(np.uint32), a_s.view(np.uint32))
    assert np.array_equal(host(askm.t).view(np.uint32), orc.scale_to_kmajor(a_s).view(np.uint32))
    assert_tol(bf16_bits_to_f64(host(out.t)), orc.gemm_ref(a, a_s, wq, ws), f"pattern M{M}N{N}K{K}")
