"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

* libfp8q.so loads and exports every function include/fp8q.h declares;
* argument validation returns the documented status before anything is
  enqueued (only arguments that fail a check before the device query are
  used here, so no call reaches the GPU even where one is present);
* fp8q_m_pad is ceil16 (page "dispatch_proj.rs", cublas_fp8_m_pad).
"""
import ctypes
import os
import re
import subprocess

import pytest

import w8a8_fp8_block_amd as fp8q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"\b(fp8q_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("fp8q_quant_act", "fp8q_scale_to_kmajor", "fp8q_gemm_blockscaled", "fp8q_proj",
              "fp8q_quant_select", "fp8q_m_pad", "fp8q_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", fp8q.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fp8q_[a-z0-9_]+)\b", out))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    lib = fp8q.lib()
    for n in _declared():
        assert getattr(lib, n) is not None


def test_m_pad():
    for m, want in ((0, 0), (1, 16), (15, 16), (16, 16), (17, 32), (25, 32), (1168, 1168),
                    (4576, 4576), (16384, 16384), (16385, 16400)):
        assert fp8q.fp8q_m_pad(m) == want


def test_version():
    assert "gfx950" in fp8q.fp8q_version()


# ---- validation: raw ctypes calls with NULL / misaligned / bad shapes ----
P = ctypes.c_void_p
BAD = P(0x1001)   # misaligned, never dereferenced (rejected first)
GOOD = P(0x1000)  # only ever passed together with an argument that fails


def _err():
    return fp8q.lib().fp8q_last_error().decode()


def test_quant_validation():
    L = fp8q.lib()
    assert L.fp8q_quant_act(None, None, None, 4, 100, None) == 2          # K % 128
    assert "K=100" in _err()
    assert L.fp8q_quant_act(None, None, None, 4, 0, None) == 2            # K == 0
    assert L.fp8q_quant_act(None, GOOD, GOOD, 4, 128, None) == 1          # NULL x
    assert "x_bf16" in _err()
    assert L.fp8q_quant_act(BAD, GOOD, GOOD, 4, 128, None) == 3           # misaligned
    assert L.fp8q_quant_act(GOOD, GOOD, None, 4, 128, None) == 1
    assert L.fp8q_quant_act_ex(GOOD, GOOD, GOOD, 4, 128, 3, None) == 6    # variant
    assert L.fp8q_quant_act_ex(GOOD, GOOD, GOOD, 4, 128, -1, None) == 6
    assert L.fp8q_quant_act(None, None, None, 1 << 20, 1 << 13, None) == 2  # > 2^32 elems
    # M == 0 is a no-op that succeeds without touching memory
    assert L.fp8q_quant_act(GOOD, GOOD, GOOD, 0, 128, None) == 0
    assert _err() == ""


def test_kmajor_validation():
    L = fp8q.lib()
    assert L.fp8q_scale_to_kmajor(GOOD, GOOD, 3, 129, None) == 2
    assert L.fp8q_scale_to_kmajor(None, GOOD, 3, 128, None) == 1
    assert L.fp8q_scale_to_kmajor(GOOD, BAD, 3, 128, None) == 3
    assert L.fp8q_scale_to_kmajor(GOOD, GOOD, 0, 128, None) == 0
    assert L.fp8q_quant_act_kmajor(GOOD, GOOD, BAD, GOOD, 3, 128, None) == 3
    assert L.fp8q_quant_act_kmajor(GOOD, GOOD, None, None, 3, 128, None) == 1
    assert L.fp8q_quant_act_kmajor(GOOD, GOOD, None, GOOD, 0, 128, None) == 0
    assert L.fp8q_quant_act_kmajor_ex(GOOD, GOOD, None, GOOD, 3, 128, 3, None) == 6   # variant
    assert L.fp8q_quant_act_kmajor_ex(GOOD, GOOD, None, GOOD, 3, 128, -1, None) == 6
    assert L.fp8q_quant_act_kmajor_ex(GOOD, GOOD, None, GOOD, 3, 100, 2, None) == 2   # K % 128
    assert L.fp8q_quant_act_kmajor_ex(GOOD, GOOD, BAD, GOOD, 3, 128, 2, None) == 3
    assert L.fp8q_quant_act_kmajor_ex(GOOD, GOOD, None, GOOD, 0, 128, 2, None) == 0


def test_gemm_validation():
    L = fp8q.lib()
    g = GOOD
    assert L.fp8q_gemm_blockscaled(g, g, g, g, g, 4, 100, 128, None) == 2   # N % 128
    assert L.fp8q_gemm_blockscaled(g, g, g, g, g, 4, 0, 128, None) == 2
    assert L.fp8q_gemm_blockscaled(g, g, g, g, g, 4, 128, 130, None) == 2   # K % 128
    assert L.fp8q_gemm_blockscaled(g, g, None, g, g, 4, 128, 128, None) == 1
    assert L.fp8q_gemm_blockscaled(g, g, g, g, BAD, 4, 128, 128, None) == 3
    assert L.fp8q_gemm_blockscaled_ex(g, g, g, g, g, 4, 128, 128, 6, None) == 6
    assert L.fp8q_gemm_blockscaled_ex(g, g, g, g, g, 4, 128, 128, -1, None) == 6
    assert L.fp8q_gemm_blockscaled(g, g, g, g, g, 0, 128, 128, None) == 0
    assert L.fp8q_proj(g, g, g, g, g, g, None, 4, 128, 128, None) == 1
    assert "act_scale_km_scratch" in _err()
    assert L.fp8q_proj(g, g, g, g, g, g, g, 4, 128, 100, None) == 2
    assert L.fp8q_proj(g, g, g, g, g, g, g, 0, 128, 128, None) == 0


def test_gemm_select():
    """Auto GEMM choice: skinny kernel up to 64 rows (and up to 128 rows when
    N <= 8192), 128x128 tiles below 129 rows; from 129 rows on the kernel with
    fewer rounds of workgroups on 256 CUs (ping-pong: tiles of 256x128 in
    rounds of 256; 128x128: workgroups in rounds of 512, a last round of at
    most 256 counting half), ties to the ping-pong kernel; bad N/K -> -1 (pure
    host function).  The expected values are the faster kernel measured at
    each of these shapes."""
    sel = fp8q.fp8q_gemm_select
    for M, want in ((1, 2), (16, 2), (25, 2), (64, 2), (65, 2), (128, 2), (129, 1), (511, 1),
                    (512, 1), (768, 1), (1024, 5), (1168, 5), (1536, 5), (2047, 1), (2048, 1),
                    (3072, 5), (4576, 5), (16384, 5)):
        assert sel(M, 5120, 17408, 256) == want, M
    for M, want in ((64, 2), (65, 1), (128, 1), (129, 5), (192, 5), (256, 5), (320, 1), (384, 1),
                    (448, 1), (511, 1), (640, 1), (768, 5), (1024, 1), (1168, 5), (1536, 1), (2048, 1),
                    (3072, 1), (4576, 5)):
        assert sel(M, 17408, 5120, 256) == want, M
    for M, want in ((768, 5), (1024, 5), (1168, 5), (1536, 1), (2048, 1), (3072, 1), (4576, 1)):
        assert sel(M, 6144, 5120, 256) == want, M
    assert sel(128, 8192, 5120, 256) == 2
    assert sel(128, 8320, 5120, 256) == 1
    assert sel(64, 100, 128, 256) == -1
    assert sel(64, 128, 0, 256) == -1
    assert sel(640, 128, 128, 0) == -1


def _rounds_rule(M, N, cus):
    """The documented round-count rule from 129 rows on, in half rounds."""
    nt = N // 128
    t_pp, t_128 = (M + 255) // 256 * nt, (M + 127) // 128 * nt
    c_pp = 2 * -(-t_pp // cus)
    tail = t_128 % (2 * cus)
    c_128 = 2 * (t_128 // (2 * cus)) + (0 if tail == 0 else 2 if tail > cus else 1)
    return 5 if c_pp <= c_128 else 1


def test_gemm_select_follows_the_cu_count():
    """The kernel choice counts rounds of workgroups on the device's own CUs.
    Hand-worked cases at N = 5120 (40 column tiles): M = 1024 on 128 CUs has
    160 ping-pong tiles (2 rounds = 4 half rounds) against 320 128x128
    workgroups (one round of 256 and a light tail of 64 = 3 half rounds):
    kernel 1, where 256 CUs take kernel 5; M = 4576 on 128 CUs: 720 tiles =
    12 half rounds against 1440 workgroups = 5 rounds + 160 > 128 = 12: a tie,
    kernel 5.  A 32-CU partition of the device: M = 640 at N = 17408 (136
    tiles): 3 x 136 = 408 ping-pong tiles (13 rounds) against 5 x 136 = 680
    workgroups (10 rounds + 40): kernel 1 (25 half rounds)."""
    sel = fp8q.fp8q_gemm_select
    assert sel(1024, 5120, 17408, 256) == 5 and sel(1024, 5120, 17408, 128) == 1
    assert sel(4576, 5120, 17408, 128) == 5
    assert sel(640, 17408, 5120, 32) == 1
    for cus in (32, 80, 128, 200, 256, 304):
        for N in (5120, 6144, 17408):
            for M in (129, 200, 256, 300, 512, 640, 1000, 1168, 2048, 3000, 4576, 9999):
                assert sel(M, N, 5120, cus) == _rounds_rule(M, N, cus), (M, N, cus)
    # below the round rule's range the CU count does not matter
    for cus in (32, 256):
        assert sel(64, 5120, 17408, cus) == 2 and sel(100, 17408, 5120, cus) == 1


def test_selectors_default_to_a_full_device_without_one():
    """Without a HIP device (this host) the device-free queries assume the
    256 CUs of a full MI355X; with one they use its CU count."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present: the queries use its CU count")
    for M, N, K in ((1024, 5120, 17408), (300, 6144, 5120), (65, 5120, 17408)):
        assert fp8q.fp8q_gemm_select(M, N, K) == fp8q.fp8q_gemm_select(M, N, K, 256)
        assert fp8q.fp8q_gemm_splitk_select(M, N, K) == fp8q.fp8q_gemm_splitk_select(M, N, K, 256)


def test_proj_quant_fused():
    """fp8q_proj fuses the relayout into the quantizer up to 2^19 scale groups."""
    assert fp8q.fp8q_proj_quant_fused(16, 5120)
    assert fp8q.fp8q_proj_quant_fused(1168, 17408)          # 158848 groups
    assert fp8q.fp8q_proj_quant_fused(4576, 6144)           # 219648 groups
    assert fp8q.fp8q_proj_quant_fused(13107, 5120)          # 524280 groups
    assert not fp8q.fp8q_proj_quant_fused(13108, 5120)      # 524320 groups
    assert not fp8q.fp8q_proj_quant_fused(4576, 17408)      # 622336 groups


def test_rowscaled_and_dequant_validation():
    L = fp8q.lib()
    g = GOOD
    assert L.fp8q_gemm_rowscaled(g, g, g, g, g, 4, 100, 128, None) == 2      # N % 128
    assert L.fp8q_gemm_rowscaled(g, g, g, None, g, 4, 128, 128, None) == 1   # NULL row scales
    assert "w_scale_row" in _err()
    assert L.fp8q_gemm_rowscaled_ex(g, g, g, g, g, 4, 128, 128, 6, None) == 6
    assert L.fp8q_gemm_rowscaled(g, g, g, g, g, 0, 128, 128, None) == 0
    assert L.fp8q_proj_rowscaled(g, g, g, g, g, g, None, 4, 128, 128, None) == 1
    assert L.fp8q_proj_rowscaled(g, g, g, g, g, g, g, 0, 128, 128, None) == 0
    # dequant: per_row 0/1 only; K multiple of 128 (blocks) or 16 (rows); any N
    assert L.fp8q_dequant_fp8_bf16(g, g, g, 4, 128, 2, None) == 6
    assert L.fp8q_dequant_fp8_bf16(g, g, g, 4, 80, 0, None) == 2
    assert L.fp8q_dequant_fp8_bf16(g, g, g, 4, 72, 1, None) == 2
    assert L.fp8q_dequant_fp8_bf16(g, g, None, 4, 80, 1, None) == 1
    assert L.fp8q_dequant_fp8_bf16(g, BAD, g, 4, 80, 1, None) == 3
    assert L.fp8q_dequant_fp8_bf16(g, g, g, 0, 80, 1, None) == 0


def test_gemm_bf16_validation():
    L = fp8q.lib()
    g = GOOD
    assert L.fp8q_gemm_bf16(g, g, g, 4, 128, 96, None) == 2     # K % 64
    assert L.fp8q_gemm_bf16(g, g, g, 4, 100, 128, None) == 2    # N % 128
    assert L.fp8q_gemm_bf16(g, None, g, 4, 128, 128, None) == 1
    assert L.fp8q_gemm_bf16(g, g, BAD, 4, 128, 128, None) == 3
    assert L.fp8q_gemm_bf16(g, g, g, 0, 128, 128, None) == 0
    assert L.fp8q_gemm_bf16(None, None, None, 1 << 16, 128, 1 << 15, None) == 2  # M*K*2 >= 2^32


def test_ffn_select_and_workspace():
    assert fp8q.fp8q_ffn_select(16, 5120, 17408) == 2
    assert fp8q.fp8q_ffn_select(32, 5120, 17408) == 2
    assert fp8q.fp8q_ffn_select(33, 5120, 17408) == 2
    assert fp8q.fp8q_ffn_select(64, 5120, 17408) == 2
    assert fp8q.fp8q_ffn_select(65, 5120, 17408) == 1
    assert fp8q.fp8q_ffn_select(4576, 5120, 17408) == 1
    assert fp8q.fp8q_ffn_select(16, 5000, 17408) == -1
    M, H, I = 4576, 5120, 17408
    Mp = fp8q.fp8q_m_pad(M)

    def a256(v):
        return (v + 255) // 256 * 256

    base = (a256(M * H) + a256(M * H // 128 * 4) + a256(Mp * H // 128 * 4) + a256(M * I)
            + a256(Mp * I // 128 * 4))
    # the down projection (N = H = 5120, K = I = 17408) at M = 4576: the
    # single-pass 256x128 kernel (no stream-K, no split), no extra workspace
    assert fp8q.fp8q_gemm_streamk_select(M, H, I) == 0
    assert fp8q.fp8q_gemm_splitk_workspace_bytes(M, H, I, 0) == 0
    assert fp8q.fp8q_ffn_workspace_bytes(M, H, I, 1) == base
    assert fp8q.fp8q_ffn_workspace_bytes(M, H, I, 2) == base + 2 * a256(2 * M * I)
    assert fp8q.fp8q_ffn_workspace_bytes(M, H, I, 0) == base
    assert fp8q.fp8q_ffn_workspace_bytes(16, H, I, 0) == fp8q.fp8q_ffn_workspace_bytes(16, H, I, 2)
    assert fp8q.fp8q_ffn_workspace_bytes(64, H, I, 0) == fp8q.fp8q_ffn_workspace_bytes(64, H, I, 2)
    assert fp8q.fp8q_ffn_workspace_bytes(65, H, I, 0) == fp8q.fp8q_ffn_workspace_bytes(65, H, I, 1)
    assert fp8q.fp8q_ffn_workspace_bytes(M, H, I, 3) == 0
    assert fp8q.fp8q_ffn_workspace_bytes(M, 100, I, 1) == 0


def test_ffn_validation():
    L = fp8q.lib()
    g = GOOD
    w = [g] * 6
    # fp8q_silu_mul_quant
    assert L.fp8q_silu_mul_quant(g, g, g, g, 4, 100, None) == 2
    assert L.fp8q_silu_mul_quant(g, None, g, g, 4, 128, None) == 1
    assert L.fp8q_silu_mul_quant(g, g, BAD, g, 4, 128, None) == 3
    assert L.fp8q_silu_mul_quant(g, g, g, g, 0, 128, None) == 0
    # fp8q_ffn_gate_up
    assert L.fp8q_ffn_gate_up(g, g, g, g, g, g, g, g, 4, 100, 256, None) == 2
    assert L.fp8q_ffn_gate_up(g, g, g, g, g, g, g, g, 4, 256, 200, None) == 2
    assert L.fp8q_ffn_gate_up(g, g, g, g, None, g, g, g, 4, 256, 256, None) == 1
    assert L.fp8q_ffn_gate_up(g, g, g, g, g, g, g, BAD, 4, 256, 256, None) == 3
    assert L.fp8q_ffn_gate_up(g, g, g, g, g, g, g, g, 0, 256, 256, None) == 0
    assert L.fp8q_ffn_gate_up(g, g, g, g, g, g, g, g, 1 << 16, 1 << 16, 256, None) == 2
    # fp8q_ffn
    need = fp8q.fp8q_ffn_workspace_bytes(8, 256, 384, 1)
    assert L.fp8q_ffn(g, *w, g, g, need, 8, 256, 384, 3, None) == 6
    assert L.fp8q_ffn(g, *w, g, g, need, 8, 256, 384, -1, None) == 6
    assert L.fp8q_ffn(g, *w, g, g, need, 8, 250, 384, 0, None) == 2
    assert L.fp8q_ffn(g, g, g, g, g, None, g, g, g, need, 8, 256, 384, 0, None) == 1
    assert L.fp8q_ffn(g, *w, BAD, g, need, 8, 256, 384, 0, None) == 3
    assert L.fp8q_ffn(g, *w, g, None, need, 8, 256, 384, 1, None) == 1
    assert L.fp8q_ffn(g, *w, g, g, need - 1, 8, 256, 384, 1, None) == 2
    assert b"workspace" in L.fp8q_last_error()
    assert L.fp8q_ffn(g, *w, g, g, need, 8, 256, 384, 2, None) == 2  # variant 2 needs more
    assert L.fp8q_ffn(g, *w, g, None, 0, 0, 256, 384, 0, None) == 0  # M == 0: nothing to do


def test_splitk_validation():
    L = fp8q.lib()
    g = GOOD
    # fp8q_gemm_blockscaled_splitk(a, as, w, ws, out, work, bytes, M, N, K, splits, stream)
    assert L.fp8q_gemm_blockscaled_splitk(g, g, g, g, g, g, 1 << 20, 4, 100, 256, 2, None) == 2
    assert L.fp8q_gemm_blockscaled_splitk(g, g, g, g, g, g, 1 << 20, 4, 128, 200, 2, None) == 2
    assert L.fp8q_gemm_blockscaled_splitk(g, g, None, g, g, g, 1 << 20, 4, 128, 256, 2, None) == 1
    assert L.fp8q_gemm_blockscaled_splitk(g, g, g, g, BAD, g, 1 << 20, 4, 128, 256, 2, None) == 3
    # split counts: 1 and more than K/128 (or 64) are rejected
    assert L.fp8q_gemm_blockscaled_splitk(g, g, g, g, g, g, 1 << 20, 4, 128, 256, 1, None) == 6
    assert L.fp8q_gemm_blockscaled_splitk(g, g, g, g, g, g, 1 << 20, 4, 128, 256, 3, None) == 6
    assert "splits=3" in _err()
    assert L.fp8q_gemm_blockscaled_splitk(g, g, g, g, g, g, 1 << 30, 4, 128, 128 * 80, 65,
                                          None) == 6
    # workspace: NULL, misaligned, too small
    need = fp8q.fp8q_gemm_splitk_workspace_bytes(4, 128, 256, 2)
    assert need == 2 * 4 * 128 * 4
    assert L.fp8q_gemm_blockscaled_splitk(g, g, g, g, g, None, need, 4, 128, 256, 2, None) == 1
    assert L.fp8q_gemm_blockscaled_splitk(g, g, g, g, g, BAD, need, 4, 128, 256, 2, None) == 3
    assert L.fp8q_gemm_blockscaled_splitk(g, g, g, g, g, g, need - 1, 4, 128, 256, 2, None) == 2
    assert "workspace" in _err()
    # M == 0: nothing to do, no workspace needed
    assert L.fp8q_gemm_blockscaled_splitk(g, g, g, g, g, None, 0, 0, 128, 256, 2, None) == 0


def test_splitk_noalloc_validation():
    """The allocation-free split-K entry point validates like the workspace
    one and refuses partials past its static scratch before the device is
    touched (the sizes here assume no device: 256 CUs)."""
    L = fp8q.lib()
    g = GOOD
    assert L.fp8q_gemm_blockscaled_splitk_noalloc(g, g, g, g, g, 4, 100, 256, 2, None) == 2  # N
    assert L.fp8q_gemm_blockscaled_splitk_noalloc(g, g, g, g, None, 4, 128, 256, 2, None) == 1
    assert L.fp8q_gemm_blockscaled_splitk_noalloc(g, g, g, g, g, 4, 128, 256, 1, None) == 6
    assert L.fp8q_gemm_blockscaled_splitk_noalloc(g, g, g, g, g, 4, 128, 256, 3, None) == 6
    assert L.fp8q_gemm_blockscaled_splitk_noalloc(g, g, g, g, g, 0, 128, 256, 2, None) == 0
    # 3 * 600 * 5120 * 4 = 36.9 MB of partials > 32 MiB
    assert L.fp8q_gemm_blockscaled_splitk_noalloc(g, g, g, g, g, 600, 5120, 17408, 3, None) == 2
    assert "static scratch" in _err()
    # the largest automatic split that fits: 3 * 512 * 5120 * 4 = 31.5 MB
    assert 3 * 512 * 5120 * 4 <= fp8q.NOALLOC_SCRATCH_BYTES == 32 << 20


def test_splitk_workspace_bytes():
    ws = fp8q.fp8q_gemm_splitk_workspace_bytes
    assert ws(300, 512, 2048, 5) == 5 * 300 * 512 * 4
    assert ws(300, 512, 2048, 1) == 0
    assert ws(300, 512, 2048, 17) == 0          # more splits than K blocks
    assert ws(300, 500, 2048, 2) == 0           # N % 128
    assert ws(300, 512, 0, 2) == 0
    for M, N, K in ((512, 5120, 17408), (200, 6144, 5120), (4576, 5120, 17408), (16, 6144, 5120)):
        s = fp8q.fp8q_gemm_splitk_select(M, N, K)
        if fp8q.fp8q_gemm_streamk_select(M, N, K) == 1:
            assert ws(M, N, K, 0) == 256 * 64 + 256 * 131072   # flags + partials, 256 CUs
        else:
            assert ws(M, N, K, 0) == (0 if s < 2 else s * M * N * 4)


def test_splitk_select():
    """Split count above 64 rows, outside the 256x128 kernel's range, with
    c = min(floor(K/1280), 6): min(floor(256 / tiles), c) if at least 2,
    else min(floor(512 / tiles), c), 1 below 2; from 8 to 64 rows, where the
    decode kernel does not take the shape, the most splits, at most c, whose
    skinny column ranges hold at most 96 columns (up to 32 rows) or 64
    (33-64 rows), else from 24 rows the tiled count; 0 for a bad N or K."""
    def sel(M, N, K):
        return fp8q.fp8q_gemm_splitk_select(M, N, K, 256)
    for M, want in ((1, 1), (7, 1), (8, 4), (16, 4), (32, 4), (33, 3), (64, 3), (65, 6), (128, 6), (129, 3),
                    (256, 3), (257, 2), (384, 2), (385, 3), (512, 3), (513, 2), (768, 2), (769, 1), (1168, 1),
                    (2048, 1)):
        assert sel(M, 5120, 17408) == want, M
    for M, want in ((8, 1), (32, 1), (33, 2), (64, 2), (65, 4), (256, 2), (384, 3), (512, 2), (640, 2), (768, 1)):
        assert sel(M, 6144, 5120) == want, M      # the decode kernel up to 32 rows: no split
    for M, want in ((16, 1), (23, 1), (24, 3), (33, 3), (64, 3), (65, 3), (128, 3), (129, 1)):
        assert sel(M, 17408, 5120) == want, M   # skinny ranges too wide: the tiled count from 24 rows
    assert sel(25, 6144, 8192) == 4        # 96 columns a workgroup
    # on 128 CUs: fewer workgroups a split, so fewer splits keep the ranges
    # within 96 / 64 columns; the decode kernel's slices no longer fit LDS
    s128 = lambda M, N, K: fp8q.fp8q_gemm_splitk_select(M, N, K, 128)
    assert s128(16, 5120, 17408) == 2      # 64 workgroups of 80 columns
    assert s128(48, 5120, 17408) == 3      # no skinny count fits 64 columns: the tiled count
    assert s128(16, 6144, 5120) == 2       # 48 columns a CU exceed the decode kernel's 32
    assert s128(4, 5120, 17408) == 1
    assert sel(300, 128, 2560) == 2        # K/1280 = 2 caps it
    assert sel(300, 128, 2432) == 1        # fewer than 20 K blocks: no split
    assert sel(4576, 5120, 17408) == 1     # the 256x128 kernel's pick: no split
    assert sel(4096, 128, 17408) == 6      # 32 128x128 tiles: six splits
    assert sel(100, 100, 1280) == 0
    assert sel(100, 128, 0) == 0


def test_splitk_select_follows_the_cu_count():
    """The split counts are sized to the device's CUs: at N = 5120, K = 17408
    (40 column tiles, at most 6 splits), M = 65 takes floor(128 / 40) = 3
    splits on 128 CUs (one workgroup per CU) and 6 on 256; M = 300 (120
    tiles) takes floor(256 / 120) = 2 on 128 CUs (two per CU) and on 304 CUs
    floor(304 / 120) = 2; M = 129 (80 tiles) on 32 CUs: floor(64 / 80) = 0,
    no split."""
    sel = fp8q.fp8q_gemm_splitk_select
    assert sel(65, 5120, 17408, 128) == 3 and sel(65, 5120, 17408, 256) == 6
    assert sel(300, 5120, 17408, 128) == 2 and sel(300, 5120, 17408, 304) == 2
    assert sel(129, 5120, 17408, 32) == 1
    assert sel(65, 5120, 17408, 0) == 0


def test_splitk_select_small_m_is_total():
    """Up to 64 rows, over odd and extreme CU counts: the automatic count is
    1 or lies in [2, min(K/1280, 6)], and no shape splits below 8 rows."""
    sel = fp8q.fp8q_gemm_splitk_select
    for cus in (1, 7, 32, 128, 256, 304, 1024):
        for N in (128, 1024, 5120, 6144, 17408, 28672):
            for K in (1280, 5120, 17408):
                cap = min(K // 1280, 6)
                for M in range(1, 65):
                    s = sel(M, N, K, cus)
                    assert s == 1 or 2 <= s <= cap, (M, N, K, cus, s)
                    if M < 8:
                        assert s == 1, (M, N, K, cus, s)


def test_ffn_workspace_holds_split_partials():
    H, I = 5120, 17408
    for M in (300, 512, 1168):
        s = fp8q.fp8q_gemm_splitk_select(M, H, I)
        extra = s * M * H * 4 if s >= 2 else 0
        Mp = fp8q.fp8q_m_pad(M)

        def a256(v):
            return (v + 255) // 256 * 256

        base = (a256(M * H) + a256(M * H // 128 * 4) + a256(Mp * H // 128 * 4) + a256(M * I)
                + a256(Mp * I // 128 * 4))
        assert fp8q.fp8q_ffn_workspace_bytes(M, H, I, 1) == base + a256(extra), M
        assert fp8q.fp8q_ffn_workspace_bytes(M, H, I, 2) == base + 2 * a256(2 * M * I) + a256(extra)


def test_proj_splitk_validation():
    L = fp8q.lib()
    g = GOOD
    M, N, K = 200, 1024, 5120
    assert fp8q.fp8q_gemm_splitk_select(M, N, K) == 4
    need = fp8q.fp8q_gemm_splitk_workspace_bytes(M, N, K, 0)
    assert need == 4 * M * N * 4
    # fp8q_proj_splitk(x, w, ws, out, aq, as, askm, work, bytes, M, N, K, stream)
    assert L.fp8q_proj_splitk(g, g, g, g, g, g, g, g, need - 1, M, N, K, None) == 2
    assert "workspace" in _err()
    assert L.fp8q_proj_splitk(g, g, g, g, g, g, g, None, need, M, N, K, None) == 1
    assert L.fp8q_proj_splitk(g, g, g, g, g, g, g, BAD, need, M, N, K, None) == 3
    assert L.fp8q_proj_splitk(g, g, g, g, g, g, g, g, need, M, N, 100, None) == 2
    assert L.fp8q_proj_splitk(g, g, g, g, g, g, g, None, 0, 0, N, K, None) == 0


def test_shader_clock_pairs_stamps_by_cu():
    """fp8q.shader_clock_ghz pairs the two stamps of the same (XCD, CU) (HW_ID
    bits 8-15) and takes d(shader counter) / d(100 MHz counter): a CU seen
    only once is ignored, and an XCD's clock is the median over its CUs."""
    import numpy as np
    before = np.array([[0, 0x0100, 1000, 10], [0, 0x0200, 50000, 10], [1, 0x0305, 7, 3],
                       [2, 0x0100, 0, 0]], dtype=np.int64)
    after = np.array([[0, 0x0100, 1000 + 1800, 110], [0, 0x0210, 50000 + 2000, 110],
                      [1, 0x0301, 7 + 2100, 103], [3, 0x0100, 5, 5]], dtype=np.int64)
    per, pairs = fp8q.shader_clock_ghz(before, after)
    assert pairs == 3 and set(per) == {0, 1}
    assert abs(per[1] - 2.1) < 1e-12                   # 2100 ticks in 100 * 10 ns
    assert abs(per[0] - (1.8 + 2.0) / 2) < 1e-12       # two CUs of XCD 0


def test_streamk_select():
    """Stream-K from 512 rows where a plan exists (more 256x128 tiles than
    CUs, not a multiple of them, the CU count a multiple of 8, K >= 256) and
    is predicted 10% shorter than the ping-pong kernel's last round.  The
    decisions follow graph-timed measurements on 256 CUs: stream-K 13%
    faster at M = 1792, N = 5120, K = 17408 (280 tiles, 24 in the last
    round); 4-7% slower at the two prefill projections (720 and 680 tiles,
    most CUs busy in the last round); no faster at N = 8448, K = 8192 and at
    N = 4224, K = 17408."""
    sel = fp8q.fp8q_gemm_streamk_select
    assert sel(1792, 5120, 17408, 256) == 1
    assert sel(2560, 6656, 17408, 256) == 1      # 520 tiles: two rounds + 8
    assert sel(1792, 5120, 17408, 240) == 1      # 280 tiles on 240 CUs: one round + 40
    assert sel(4576, 5120, 17408, 256) == 0 and sel(1168, 17408, 5120, 256) == 0
    assert sel(2048, 8448, 8192, 256) == 0 and sel(3072, 4224, 17408, 256) == 0
    assert sel(16384, 5120, 17408, 256) == 0     # 2560 tiles: 10 whole rounds
    assert sel(1024, 5120, 17408, 256) == 0      # 160 tiles: fewer than the CUs
    assert sel(1792, 5120, 17408, 304) == 0      # 280 tiles: fewer than the CUs
    assert sel(1792, 5120, 17408, 252) == 0      # not a multiple of 8 workgroups
    assert sel(1792, 5120, 1024, 256) == 0       # short K: the partial reads dominate
    assert sel(500, 40960, 17408, 256) == 0      # under 512 rows
    assert sel(4576, 5000, 17408, 256) == -1 and sel(4576, 5120, 17408, 0) == -1


def test_streamk_workspace_bytes():
    ws = fp8q.fp8q_gemm_streamk_workspace_bytes
    assert ws(256) == 256 * 64 + 256 * 131072     # flags, then one partial slot a workgroup
    assert ws(8) == 512 + 8 * 131072              # 8 waves x 8 bytes of flags a workgroup
    assert ws(24) == 1536 + 24 * 131072
    assert ws(12) == 0                            # not a multiple of 8


def test_streamk_validation():
    """The explicit stream-K entry point: argument checks, then the plan,
    then the workspace, all before the device is touched."""
    L = fp8q.lib()
    g = GOOD
    # fp8q_gemm_blockscaled_streamk(a, as, w, ws, out, work, bytes, M, N, K, workgroups, stream)
    f = L.fp8q_gemm_blockscaled_streamk
    assert f(g, g, g, g, g, g, 1 << 30, 300, 100, 1024, 8, None) == 2        # N % 128
    assert f(g, g, None, g, g, g, 1 << 30, 300, 128, 1024, 8, None) == 1     # NULL operand
    assert f(g, g, g, g, BAD, g, 1 << 30, 300, 128, 1024, 8, None) == 3      # misaligned
    assert f(g, g, g, g, g, g, 1 << 30, 300, 1664, 1024, 12, None) == 6      # workgroups % 8
    assert "workgroups=12" in _err()
    # plans: 2 x 5 = 10 tiles on 8 workgroups; 8 tiles (a multiple); one K block
    assert f(g, g, g, g, g, None, 0, 300, 640, 1024, 8, None) == 1           # NULL workspace
    assert f(g, g, g, g, g, g, 1 << 30, 300, 1024, 1024, 8, None) == 2
    assert "no stream-K plan" in _err()
    assert f(g, g, g, g, g, g, 1 << 30, 300, 640, 128, 8, None) == 2
    assert f(g, g, g, g, g, g, 1 << 30, 256, 1024, 1024, 8, None) == 2      # 8 tiles: T <= C
    need = fp8q.fp8q_gemm_streamk_workspace_bytes(8)
    assert f(g, g, g, g, g, BAD, need, 300, 640, 1024, 8, None) == 3
    assert f(g, g, g, g, g, g, need - 1, 300, 640, 1024, 8, None) == 2
    assert "workspace" in _err()
    assert f(g, g, g, g, g, None, 0, 0, 640, 1024, 8, None) == 0            # M == 0


def test_gemm_kernel_name():
    """The kernel names the benchmark line and the profiles use, as a kernel
    trace shows them (no device here: 256 CUs assumed)."""
    name = fp8q.fp8q_gemm_kernel_name
    # decode widths at N = 6144, K = 5120: 24 columns a workgroup, 5 K blocks a wave
    assert name(16, 6144, 5120) == "gemm_decode_kernel<1, 5, false>"
    assert name(25, 6144, 5120) == "gemm_decode_kernel<2, 5, false>"
    assert name(16, 256, 512) == "gemm_decode_kernel<1, 2, false>"
    # wider slices (68 columns), more rows, or longer K: the fragment-layout kernel
    assert name(16, 17408, 5120) == "gemm_skinny_kernel<1, 6, 8, 2, false>"
    assert name(64, 6144, 5120) == "gemm_skinny_kernel<4, 2, 8, 2, false>"
    assert name(16, 5120, 17408).startswith("gemm_skinny_kernel<")
    assert name(4576, 5120, 17408) == "gemm_pp_kernel<3, false, false>"
    assert name(300, 512, 896) == "gemm_tiled_kernel<128, 128, 2, 2, 2, false, false>"
    assert name(4576, 5120, 17408, 1) == "gemm_tiled_kernel<128, 128, 2, 2, 2, false, false>"
    assert name(16, 100, 512) == "" and name(16, 128, 512, 9) == ""
