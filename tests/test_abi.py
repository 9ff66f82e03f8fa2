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
    N <= 8192), 128x128 tiles below 512 rows; from 512 rows on the kernel with
    fewer rounds of workgroups on 256 CUs (ping-pong: tiles of 256x128 in
    rounds of 256; 128x128: workgroups in rounds of 512, a last round of at
    most 256 counting half), ties to the ping-pong kernel; bad N/K -> -1 (pure
    host function).  The expected values are the faster kernel measured at
    each of these shapes."""
    for M, want in ((1, 2), (16, 2), (25, 2), (64, 2), (65, 2), (128, 2), (129, 1), (511, 1),
                    (512, 1), (768, 1), (1024, 5), (1168, 5), (1536, 5), (2047, 1), (2048, 1),
                    (3072, 5), (4576, 5), (16384, 5)):
        assert fp8q.fp8q_gemm_select(M, 5120, 17408) == want, M
    for M, want in ((64, 2), (65, 1), (128, 1), (640, 1), (768, 5), (1024, 1), (1168, 5),
                    (1536, 1), (2048, 1), (3072, 1), (4576, 5)):
        assert fp8q.fp8q_gemm_select(M, 17408, 5120) == want, M
    for M, want in ((768, 5), (1024, 5), (1168, 5), (1536, 1), (2048, 1), (3072, 1), (4576, 1)):
        assert fp8q.fp8q_gemm_select(M, 6144, 5120) == want, M
    assert fp8q.fp8q_gemm_select(128, 8192, 5120) == 2
    assert fp8q.fp8q_gemm_select(128, 8320, 5120) == 1
    assert fp8q.fp8q_gemm_select(64, 100, 128) == -1
    assert fp8q.fp8q_gemm_select(64, 128, 0) == -1


def test_proj_quant_fused():
    """fp8q_proj fuses the relayout into the quantizer up to 2^17 scale groups."""
    assert fp8q.fp8q_proj_quant_fused(16, 5120)
    assert fp8q.fp8q_proj_quant_fused(1168, 5120)           # 46720 groups
    assert not fp8q.fp8q_proj_quant_fused(1168, 17408)      # 158848 groups
    assert fp8q.fp8q_proj_quant_fused(3276, 5120)           # 131040 groups
    assert not fp8q.fp8q_proj_quant_fused(3277, 5120)       # 131080 groups
    assert not fp8q.fp8q_proj_quant_fused(4576, 17408)


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
    assert fp8q.fp8q_ffn_select(33, 5120, 17408) == 1
    assert fp8q.fp8q_ffn_select(64, 5120, 17408) == 1
    assert fp8q.fp8q_ffn_select(4576, 5120, 17408) == 1
    assert fp8q.fp8q_ffn_select(16, 5000, 17408) == -1
    M, H, I = 4576, 5120, 17408
    Mp = fp8q.fp8q_m_pad(M)

    def a256(v):
        return (v + 255) // 256 * 256

    base = (a256(M * H) + a256(M * H // 128 * 4) + a256(Mp * H // 128 * 4) + a256(M * I)
            + a256(Mp * I // 128 * 4))
    assert fp8q.fp8q_ffn_workspace_bytes(M, H, I, 1) == base
    assert fp8q.fp8q_ffn_workspace_bytes(M, H, I, 2) == base + 2 * a256(2 * M * I)
    assert fp8q.fp8q_ffn_workspace_bytes(M, H, I, 0) == base
    assert fp8q.fp8q_ffn_workspace_bytes(16, H, I, 0) == fp8q.fp8q_ffn_workspace_bytes(16, H, I, 2)
    assert fp8q.fp8q_ffn_workspace_bytes(33, H, I, 0) == fp8q.fp8q_ffn_workspace_bytes(33, H, I, 1)
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


def test_splitk_workspace_bytes():
    ws = fp8q.fp8q_gemm_splitk_workspace_bytes
    assert ws(300, 512, 2048, 5) == 5 * 300 * 512 * 4
    assert ws(300, 512, 2048, 1) == 0
    assert ws(300, 512, 2048, 17) == 0          # more splits than K blocks
    assert ws(300, 500, 2048, 2) == 0           # N % 128
    assert ws(300, 512, 0, 2) == 0
    for M, N, K in ((512, 5120, 17408), (200, 6144, 5120), (4576, 5120, 17408), (16, 6144, 5120)):
        s = fp8q.fp8q_gemm_splitk_select(M, N, K)
        assert ws(M, N, K, 0) == (0 if s < 2 else s * M * N * 4)


def test_splitk_select():
    """Split count above 64 rows, outside the 256x128 kernel's range, with
    c = min(floor(K/1280), 6): min(floor(256 / tiles), c) if at least 2,
    else min(floor(512 / tiles), c), 1 below 2; 0 for a bad N or K."""
    sel = fp8q.fp8q_gemm_splitk_select
    for M, want in ((16, 1), (64, 1), (65, 6), (128, 6), (129, 3), (256, 3), (257, 2), (384, 2),
                    (385, 3), (512, 3), (513, 2), (768, 2), (769, 1), (1168, 1), (2048, 1)):
        assert sel(M, 5120, 17408) == want, M
    for M, want in ((65, 4), (256, 2), (384, 3), (512, 2), (640, 2), (768, 1)):
        assert sel(M, 6144, 5120) == want, M
    for M, want in ((65, 3), (128, 3), (129, 1)):
        assert sel(M, 17408, 5120) == want, M
    assert sel(300, 128, 2560) == 2        # K/1280 = 2 caps it
    assert sel(300, 128, 2432) == 1        # fewer than 20 K blocks: no split
    assert sel(4576, 5120, 17408) == 1     # the 256x128 kernel's pick: no split
    assert sel(4096, 128, 17408) == 6      # 32 128x128 tiles: six splits
    assert sel(100, 100, 1280) == 0
    assert sel(100, 128, 0) == 0


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
