"""GPU parity of the split-K form of the block-scaled FP8 GEMM
(fp8q_gemm_blockscaled_splitk) against the oracle's fp64 block-form product,
with the same accuracy contract as the single-pass kernels (rel_rms <= 1e-3
against the bf16-rounded reference; per element |o - r| <= ulp_bf16(r) +
1e-3*RMS(r)).  Split counts that do and do not divide the K-block count,
one block per split, ragged row tiles, exact special cases that must match
bit for bit, workspace and output canaries, and run-to-run reproducibility.
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


def _splitk_gpu(orc, a, a_s, wq, ws, splits, km=None):
    M, K = a.shape
    N = wq.shape[0]
    if km is None:
        km = orc.scale_to_kmajor(a_s)
    need = fp8q.fp8q_gemm_splitk_workspace_bytes(M, N, K, splits)
    out = Guarded((M, N), torch.int16)
    work = Guarded((max(need, 16) // 4,), torch.float32, fill=0x7F) if need else None
    fp8q.fp8q_gemm_blockscaled_splitk(dev(a), dev(km), dev(wq), dev(ws), out.t,
                                      None if work is None else work.t, splits=splits)
    torch.cuda.synchronize()
    out.check_canary()
    if work is not None:
        work.check_canary()
    return bf16_bits_to_f64(host(out.t))


def _random_operands(orc, M, N, K, seed, dist="normal"):
    rng = np.random.default_rng(seed)
    v = rng.laplace(0, 1, (M, K)) if dist == "laplace" else rng.standard_normal((M, K))
    x = synth.f32_to_bf16_bits(v.astype(np.float32))
    a, a_s = orc.quant_act(x)
    wq, ws = orc.quant_weight_block(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    return a, a_s, wq, ws


# (M, N, K, splits): K blocks 7 over 2/3/7 splits (uneven ranges and one block
# each), ragged row tiles (130, 257, 300), one row, several column tiles.
@pytest.mark.parametrize("M,N,K,splits", [(130, 384, 896, 2), (130, 384, 896, 3),
                                          (130, 384, 896, 7), (1, 128, 256, 2),
                                          (257, 256, 1280, 4), (300, 512, 2048, 5),
                                          (64, 256, 640, 5), (17, 128, 4096, 8)])
def test_splitk_full(orc, M, N, K, splits):
    a, a_s, wq, ws = _random_operands(orc, M, N, K, M * 31 + N + K + splits)
    ref = orc.gemm_ref(a, a_s, wq, ws)
    log(f"splitk M={M} N={N} K={K} splits={splits}")
    assert_tol(_splitk_gpu(orc, a, a_s, wq, ws, splits), ref, f"M{M}N{N}K{K}s{splits}")


def test_splitk_auto_falls_back_without_workspace(orc):
    """splits = 0 where the selector gives 1: the single-pass automatic kernel
    runs, no workspace is needed, and the output equals fp8q_gemm_blockscaled's
    bit for bit."""
    M, N, K = 40, 256, 512
    assert fp8q.fp8q_gemm_splitk_select(M, N, K) == 1
    assert fp8q.fp8q_gemm_splitk_workspace_bytes(M, N, K, 0) == 0
    a, a_s, wq, ws = _random_operands(orc, M, N, K, 3)
    o = _splitk_gpu(orc, a, a_s, wq, ws, 0)
    km = orc.scale_to_kmajor(a_s)
    out = torch.empty((M, N), dtype=torch.int16, device="cuda")
    fp8q.fp8q_gemm_blockscaled(dev(a), dev(km), dev(wq), dev(ws), out)
    torch.cuda.synchronize()
    assert np.array_equal(o, bf16_bits_to_f64(host(out)))


def test_splitk_small_integers_exact(orc):
    """Small-integer codes and power-of-two scales: every partial sum and the
    sum of the splits' partials are exact in fp32, so the output is the bf16
    rounding of the exact value, whatever the split."""
    M, N, K = 37, 256, 1536
    G = K // 128
    rng = np.random.default_rng(4)
    a = orc.e4m3_encode(rng.integers(-3, 4, (M, K)).astype(np.float32))
    wq = orc.e4m3_encode(rng.integers(-3, 4, (N, K)).astype(np.float32))
    a_s = np.exp2(rng.integers(-2, 3, (M, G))).astype(np.float32)
    ws = np.exp2(rng.integers(-2, 3, (N // 128, G))).astype(np.float32)
    ref = orc.gemm_ref(a, a_s, wq, ws)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    want = bf16_bits_to_f64(synth.f32_to_bf16_bits(ref.astype(np.float32)))
    for splits in (2, 3, 5, 12):
        assert np.array_equal(_splitk_gpu(orc, a, a_s, wq, ws, splits), want), splits


def test_splitk_block_scale_isolation_exact(orc):
    """All codes 1.0, a_s[m,g] = 2^(m%5), w_s[nb,g] = 2^g * (nb+1): a K block
    read with another block's scale, or a split's range taken twice or not at
    all, changes the exact fp32 result and so its bf16 rounding."""
    M, N, K = 40, 384, 1024
    G = K // 128
    a = np.full((M, K), 0x38, dtype=np.uint8)
    wq = np.full((N, K), 0x38, dtype=np.uint8)
    a_s = np.array([[2.0 ** (m % 5)] * G for m in range(M)], dtype=np.float32)
    ws = np.array([[2.0 ** g * (nb + 1) for g in range(G)] for nb in range(N // 128)],
                  dtype=np.float32)
    ref = orc.gemm_ref(a, a_s, wq, ws)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)  # exact in fp32
    want = bf16_bits_to_f64(synth.f32_to_bf16_bits(ref.astype(np.float32)))
    for splits in (2, 3, 8):
        assert np.array_equal(_splitk_gpu(orc, a, a_s, wq, ws, splits), want), splits


def test_splitk_repeatable(orc):
    """Same inputs, same bits, run to run (the reduction order is fixed)."""
    a, a_s, wq, ws = _random_operands(orc, 200, 256, 2048, 9, "laplace")
    for splits in (3, 6):
        o1 = _splitk_gpu(orc, a, a_s, wq, ws, splits)
        o2 = _splitk_gpu(orc, a, a_s, wq, ws, splits)
        assert np.array_equal(o1, o2)


@pytest.mark.parametrize("M,N,K", [(512, 5120, 17408), (200, 6144, 5120), (48, 5120, 17408),
                                   (16, 5120, 17408), (25, 6144, 8192), (40, 17408, 5120)])
def test_splitk_projection_shapes_full(orc, M, N, K):
    """Medium and decode row counts at the down- and gate/up-projection
    shapes, with the automatic split count, 2 and one above the automatic
    count: all M*N outputs against the oracle.  Up to 64 rows the splits run
    the skinny kernel's split form where its column ranges hold at most 128
    columns (48 rows: 2, 3 and 4 splits of 40, 64 and 80 columns a
    workgroup; 16 rows: 2, 4 and 5, 40 to 104 columns; 25 rows at N = 6144,
    K = 8192: 2, 4 and 5), else the tiled split form (40 rows at N = 17408:
    2, 3 and 4 splits, whose skinny ranges would hold 136 columns or more)."""
    a, a_s, wq, ws = _random_operands(orc, M, N, K, M + K, "laplace")
    log(f"oracle M={M} N={N} K={K}: full fp64 product")
    ref = orc.gemm_ref(a, a_s, wq, ws)
    auto = fp8q.fp8q_gemm_splitk_select(M, N, K)
    for splits in sorted({0, 2, max(auto, 2) + 1}):
        log(f"splitk M={M} N={N} K={K} splits={splits} (auto {auto})")
        o = _splitk_gpu(orc, a, a_s, wq, ws, splits)
        assert np.all(np.isfinite(o))
        assert_tol(o, ref, f"M{M}N{N}K{K}s{splits}")


@pytest.mark.parametrize("M,N,K", [(200, 1024, 5120), (96, 6144, 5120), (40, 512, 2048),
                                   (64, 17408, 5120)])
def test_proj_splitk(orc, M, N, K):
    """fp8q_proj_splitk: the quantizer's codes and both scale layouts as
    fp8q_proj writes them (bit-exact against the oracle), the output equal bit
    for bit to fp8q_gemm_blockscaled_splitk (splits = 0) on those codes, and
    within the projection tolerance of the oracle; where the selector does not
    split (M = 40 at K = 2048: fewer than 20 K blocks) the workspace may be
    absent and the output is fp8q_proj's.  M = 64 at N = 17408 takes the
    tiled split form (3 splits)."""
    rng = np.random.default_rng(M + N)
    x = synth.f32_to_bf16_bits((rng.standard_normal((M, K)) *
                                np.exp(rng.uniform(-2, 2, (M, 1)))).astype(np.float32))
    wq, ws = orc.quant_weight_block(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    a, a_s = orc.quant_act(x)
    splits = fp8q.fp8q_gemm_splitk_select(M, N, K)
    need = fp8q.fp8q_gemm_splitk_workspace_bytes(M, N, K, 0)
    log(f"proj_splitk M={M} N={N} K={K} splits={splits}")
    out = Guarded((M, N), torch.int16)
    aq = Guarded((M, K), torch.uint8)
    asr = Guarded((M, K // 128), torch.float32)
    askm = Guarded((K // 128, synth.ceil16(M)), torch.float32, fill=0x7F)
    work = Guarded((need // 4,), torch.float32, fill=0x7F) if need else None
    fp8q.fp8q_proj_splitk(dev(x), dev(wq), dev(ws), out.t, aq.t, asr.t, askm.t,
                          None if work is None else work.t)
    torch.cuda.synchronize()
    for gd in (out, aq, asr, askm) + ((work,) if work is not None else ()):
        gd.check_canary()
    assert np.array_equal(host(aq.t), a)
    assert np.array_equal(host(asr.t).view(np.uint32), a_s.view(np.uint32))
    assert np.array_equal(host(askm.t).view(np.uint32), orc.scale_to_kmajor(a_s).view(np.uint32))
    o = bf16_bits_to_f64(host(out.t))
    if splits >= 2:
        assert np.array_equal(o, _splitk_gpu(orc, a, a_s, wq, ws, 0))
    else:
        assert need == 0
        ref_out = torch.empty((M, N), dtype=torch.int16, device="cuda")
        fp8q.fp8q_proj(dev(x), dev(wq), dev(ws), ref_out, aq.t, asr.t, askm.t)
        torch.cuda.synchronize()
        assert np.array_equal(o, bf16_bits_to_f64(host(ref_out)))
    assert_tol(o, orc.gemm_ref(a, a_s, wq, ws), f"proj_splitk M{M}N{N}K{K}")


def _streamk_gpu(orc, a, a_s, wq, ws, workgroups, repeat=1):
    """fp8q_gemm_blockscaled_streamk `repeat` times back to back into separate
    outputs (one workspace, which starts non-zero), canaries checked."""
    M, K = a.shape
    N = wq.shape[0]
    km = orc.scale_to_kmajor(a_s)
    need = fp8q.fp8q_gemm_streamk_workspace_bytes(workgroups)
    work = Guarded((need // 4,), torch.float32, fill=0x7F)
    outs = [Guarded((M, N), torch.int16) for _ in range(repeat)]
    a_d, km_d, w_d, ws_d = dev(a), dev(km), dev(wq), dev(ws)
    for o in outs:
        fp8q.fp8q_gemm_blockscaled_streamk(a_d, km_d, w_d, ws_d, o.t, work.t, workgroups)
    torch.cuda.synchronize()
    work.check_canary()
    res = []
    for o in outs:
        o.check_canary()
        res.append(bf16_bits_to_f64(host(o.t)))
    return res


# (M, N, K, workgroups C): T = ceil(M/256) * N/128 tiles, R whole rounds, Tt
# tail tiles, P pieces a tail tile.
#   256 x 1664 x 1024 on 8:  T = 13, R = 1, Tt = 5 > C/2: P = 2, the 3
#                            secondaries take the second pieces in 2 rounds
#   300 x 1152 x 8192 on 8:  T = 18, R = 2, Tt = 2: P = 4, ragged last row tile
#   256 x 1152 x 17408 on 8: T = 9, R = 1, Tt = 1: P = 5 (G = 136)
#   520 x 1280 x 2048 on 16: T = 30, R = 1, Tt = 14: P = 2 in 7 rounds, an
#                            8-row last row tile
#   1168 x 17408 x 1024 and 4576 x 5120 x 1024 on one workgroup per CU (the
#   prefill shapes at short K): 680 / 720 tiles, Tt = 168 / 208, P = 2
STREAMK_CASES = [(256, 1664, 1024, 8), (300, 1152, 8192, 8), (256, 1152, 17408, 8),
                 (520, 1280, 2048, 16), (1168, 17408, 1024, 0), (4576, 5120, 1024, 0)]


@pytest.mark.parametrize("M,N,K,C", STREAMK_CASES,
                         ids=[f"M{m}N{n}K{k}C{c}" for m, n, k, c in STREAMK_CASES])
def test_streamk_plans_full(orc, M, N, K, C):
    """The stream-K form under every kind of plan: all M*N outputs against
    the oracle, and the same bits from two more launches back to back on the
    same workspace (the flags of one call must not release the next)."""
    a, a_s, wq, ws = _random_operands(orc, M, N, K, M + N + K + C, "laplace")
    log(f"oracle M={M} N={N} K={K}")
    ref = orc.gemm_ref(a, a_s, wq, ws)
    log(f"streamk M={M} N={N} K={K} workgroups={C}")
    outs = _streamk_gpu(orc, a, a_s, wq, ws, C, repeat=3)
    assert_tol(outs[0], ref, f"streamk M{M}N{N}K{K}C{C}")
    for i, o in enumerate(outs[1:]):
        assert np.array_equal(o, outs[0]), f"stream-K launch {i + 1} differs"


def test_streamk_exact_cases(orc):
    """Codes 1.0 (0x38) and power-of-two scales: each block adds 128 *
    2^e, e in [-12, 2], and the 64 blocks' sum spans under 2^20, so every
    partial sum is exact in fp32 whatever its order: the output is the
    oracle's value rounded to bf16, bit for bit (P = 4 pieces, ragged row
    tile)."""
    M, N, K, C = 300, 1152, 8192, 8
    a = np.full((M, K), 0x38, dtype=np.uint8)
    wq = np.full((N, K), 0x38, dtype=np.uint8)
    rng = np.random.default_rng(4)
    a_s = np.ldexp(1.0, rng.integers(-6, 2, (M, K // 128))).astype(np.float32)
    ws = np.ldexp(1.0, rng.integers(-6, 2, (N // 128, K // 128))).astype(np.float32)
    out, = _streamk_gpu(orc, a, a_s, wq, ws, C)
    assert np.array_equal(out, orc.round_to_bf16(orc.gemm_ref(a, a_s, wq, ws)))


def test_streamk_graph_replay(orc):
    """A captured stream-K launch replays with the same generation number:
    each replay must wait for its own partials.  Three replays, with eager
    stream-K calls on the same workspace and a host synchronization between
    them, each checked bit for bit against the eager result."""
    M, N, K, C = 300, 1152, 8192, 8
    a, a_s, wq, ws = _random_operands(orc, M, N, K, 77)
    km = orc.scale_to_kmajor(a_s)
    a_d, km_d, w_d, ws_d = dev(a), dev(km), dev(wq), dev(ws)
    work = torch.empty((fp8q.fp8q_gemm_streamk_workspace_bytes(C) // 4,), dtype=torch.float32,
                       device="cuda")
    eager = torch.empty((M, N), dtype=torch.int16, device="cuda")
    fp8q.fp8q_gemm_blockscaled_streamk(a_d, km_d, w_d, ws_d, eager, work, C)
    torch.cuda.synchronize()
    ref = host(eager).copy()
    assert_tol(bf16_bits_to_f64(ref), orc.gemm_ref(a, a_s, wq, ws), "streamk eager")
    out = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8q.fp8q_gemm_blockscaled_streamk(a_d, km_d, w_d, ws_d, out, work, C)
    for r in range(3):
        out.fill_(0)
        log(f"streamk graph replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), ref), f"replay {r} differs from the eager result"
        other = torch.empty_like(eager)
        fp8q.fp8q_gemm_blockscaled_streamk(a_d, km_d, w_d, ws_d, other, work, C)
        torch.cuda.synchronize()
        assert np.array_equal(host(other), ref)


def test_streamk_auto_sampled(orc):
    """The automatic choice of the workspace form at a shape where it takes
    stream-K (M = 1792, N = 5120, K = 17408: 280 tiles on 256 CUs, 24 in the
    last round, P = 5): the same bits as the explicit entry point, and every
    output of 56 sampled rows (8 from each 256-row tile) against the oracle."""
    M, N, K = 1792, 5120, 17408
    if fp8q.fp8q_gemm_streamk_select(M, N, K) != 1:
        pytest.skip("the automatic choice on this device's CU count is not stream-K here")
    a, a_s, wq, ws = _random_operands(orc, M, N, K, 5)
    km = orc.scale_to_kmajor(a_s)
    need = fp8q.fp8q_gemm_splitk_workspace_bytes(M, N, K, 0)
    assert need == fp8q.fp8q_gemm_streamk_workspace_bytes(0)
    work = Guarded((need // 4,), torch.float32, fill=0x7F)
    out = Guarded((M, N), torch.int16)
    log(f"streamk auto M={M} N={N} K={K}")
    fp8q.fp8q_gemm_blockscaled_splitk(dev(a), dev(km), dev(wq), dev(ws), out.t, work.t)
    torch.cuda.synchronize()
    out.check_canary()
    work.check_canary()
    got = bf16_bits_to_f64(host(out.t))
    explicit, = _streamk_gpu(orc, a, a_s, wq, ws, 0)
    assert np.array_equal(got, explicit)
    rows = np.concatenate([t * 256 + np.random.default_rng(t).choice(256, 8, replace=False)
                           for t in range(M // 256)])
    log(f"oracle M={M} N={N} K={K}: {rows.size} rows")
    ref = orc.gemm_ref(a[rows], a_s[rows], wq, ws)
    assert_tol(got[rows], ref, f"streamk auto M{M}N{N}K{K} sampled rows")
