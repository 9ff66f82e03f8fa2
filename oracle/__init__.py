"""fp8q oracle -- TEST INFRASTRUCTURE ONLY.

ctypes wrapper around ``liboracle.so`` (built from ``fp8q_oracle.c`` with the
host C compiler).  Only ``tests/``, the smoke check and the benchmark's
CPU-baseline leg may import this package; the GPU product path never does.

Every function takes and returns numpy arrays:

* ``quant_act(x_bf16[M,K] uint16) -> (codes[M,K] uint8, scale[M,K/128] f32)``
* ``scale_to_kmajor(scale_rm[M,G] f32) -> km[G, ceil16(M)] f32``
* ``quant_weight_block(w[N,K] f32) -> (codes[N,K] uint8, scale[N/128,K/128] f32)``
* ``quant_weight_row(w[N,K] f32) -> (codes[N,K] uint8, scale[N] f32)``
* ``dequant_fp8_bf16(codes[N,K], scale) -> bf16 bits[N,K] uint16`` (either weight format)
* ``gemm_ref(a, a_s_rm, w, w_s) -> out[M,N] f64`` (w_s block-scaled 2-D or per-row 1-D)
* ``gemm_ref_at(a, a_s_rm, w, w_s, ms, ns) -> out[len] f64``
* ``gemm_bf16_ref(x_bits[M,K], w_bits[N,K]) -> out[M,N] f64`` (bf16 comparator)
* ``e4m3_decode(codes) -> f64``, ``e4m3_encode(f32) -> uint8``
* ``f64_to_bf16(v) -> bf16 bits`` (one rounding, ties to even)
* ``silu_mul(g_bits, u_bits) -> (h_bits, ambiguous)``: the FFN intermediate
* ``ffn_ref(x_bits, wg, wg_s, wu, wu_s, wd, wd_s, rows=None) -> dict``: the
  whole FFN chain (quantize x once, gate and up, SiLU * up, quantize the
  intermediate once, down)

See ``fp8q_oracle.c`` for the definitions and the passages they follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8q_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

GROUP = 128


def build(force: bool = True) -> str:
    """Compile liboracle.so with the host C compiler (no fast-math)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int64
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode_array.argtypes = [P, P, I]
    lib.oracle_e4m3_encode_array.restype = None
    lib.oracle_quant_act.argtypes = [P, P, P, I, I]
    lib.oracle_quant_act.restype = None
    lib.oracle_m_pad.argtypes = [I]
    lib.oracle_m_pad.restype = I
    lib.oracle_scale_to_kmajor.argtypes = [P, P, I, I]
    lib.oracle_scale_to_kmajor.restype = None
    lib.oracle_quant_weight_block.argtypes = [P, P, P, I, I]
    lib.oracle_quant_weight_block.restype = None
    lib.oracle_gemm_ref.argtypes = [P, P, P, P, P, I, I, I]
    lib.oracle_gemm_ref.restype = None
    lib.oracle_gemm_ref_at.argtypes = [P, P, P, P, P, P, P, I, I]
    lib.oracle_gemm_ref_at.restype = None
    lib.oracle_quant_weight_row.argtypes = [P, P, P, I, I]
    lib.oracle_quant_weight_row.restype = None
    lib.oracle_dequant_fp8_bf16.argtypes = [P, P, P, I, I, I, I, I]
    lib.oracle_dequant_fp8_bf16.restype = None
    lib.oracle_gemm_ref_geom.argtypes = [P, P, P, P, P, I, I, I, I, I, I]
    lib.oracle_gemm_ref_geom.restype = None
    lib.oracle_gemm_ref_at_geom.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I]
    lib.oracle_gemm_ref_at_geom.restype = None
    lib.oracle_f64_to_bf16_array.argtypes = [P, P, I]
    lib.oracle_f64_to_bf16_array.restype = None
    lib.oracle_silu_mul.argtypes = [P, P, P, P, I]
    lib.oracle_silu_mul.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def num_threads() -> int:
    return _load().oracle_num_threads()


def m_pad(M: int) -> int:
    return int(_load().oracle_m_pad(M))


def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib.oracle_e4m3_decode(i) for i in range(256)])
    return table[c]


def e4m3_encode(q) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float32)
    out = np.empty(q.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode_array(_p(q), _p(out), q.size)
    return out


def quant_act(x_bf16: np.ndarray):
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x.shape
    assert K % GROUP == 0
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // GROUP), dtype=np.float32)
    _load().oracle_quant_act(_p(x), _p(q), _p(s), M, K)
    return q, s


def scale_to_kmajor(scale_rm: np.ndarray) -> np.ndarray:
    s = np.ascontiguousarray(scale_rm, dtype=np.float32)
    M, G = s.shape
    km = np.empty((G, m_pad(M)), dtype=np.float32)
    _load().oracle_scale_to_kmajor(_p(s), _p(km), M, G * GROUP)
    return km


def quant_weight_block(w: np.ndarray):
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert N % GROUP == 0 and K % GROUP == 0
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty((N // GROUP, K // GROUP), dtype=np.float32)
    _load().oracle_quant_weight_block(_p(w), _p(q), _p(s), N, K)
    return q, s


def quant_weight_row(w: np.ndarray):
    """Per-row FP8 weights: codes [N,K] and scale[n] = row amax / 448."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty((N,), dtype=np.float32)
    _load().oracle_quant_weight_row(_p(w), _p(q), _p(s), N, K)
    return q, s


def weight_geometry(N: int, K: int, w_s: np.ndarray):
    """(block_n, block_k, sk) of the pages' weight-scale index
    scale[(n/block_n)*sk + k/block_k]: a 2-D [ceil(N/128), K/128] array is the
    128x128 block-scaled format, a 1-D [N] array the per-row format."""
    if w_s.ndim == 1:
        assert w_s.shape == (N,)
        return 1, K, 1
    assert w_s.shape == ((N + GROUP - 1) // GROUP, K // GROUP), w_s.shape
    return GROUP, GROUP, K // GROUP


def dequant_fp8_bf16(w: np.ndarray, w_s: np.ndarray) -> np.ndarray:
    """bf16 bit patterns [N,K] of fl32(dec(w) * scale), either weight format."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    w_s = np.ascontiguousarray(w_s, dtype=np.float32)
    N, K = w.shape
    bn, bk, sk = weight_geometry(N, K, w_s)
    out = np.empty((N, K), dtype=np.uint16)
    _load().oracle_dequant_fp8_bf16(_p(w), _p(w_s), _p(out), N, K, bn, bk, sk)
    return out


def gemm_ref(a, a_s_rm, w, w_s) -> np.ndarray:
    """fp64 block-form product; w_s block-scaled [N/128, K/128] or per-row [N]."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    a_s = np.ascontiguousarray(a_s_rm, dtype=np.float32)
    w_s = np.ascontiguousarray(w_s, dtype=np.float32)
    M, K = a.shape
    N = w.shape[0]
    assert w.shape[1] == K and a_s.shape == (M, K // GROUP)
    assert w_s.ndim == 1 or N % GROUP == 0
    bn, bk, sk = weight_geometry(N, K, w_s)
    out = np.empty((M, N), dtype=np.float64)
    _load().oracle_gemm_ref_geom(_p(a), _p(a_s), _p(w), _p(w_s), _p(out), M, N, K, bn, bk, sk)
    return out


def gemm_ref_at(a, a_s_rm, w, w_s, ms, ns) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    a_s = np.ascontiguousarray(a_s_rm, dtype=np.float32)
    w_s = np.ascontiguousarray(w_s, dtype=np.float32)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    M, K = a.shape
    N = w.shape[0]
    assert ms.shape == ns.shape
    assert (ms >= 0).all() and (ms < M).all() and (ns >= 0).all() and (ns < N).all()
    assert a_s.shape == (M, K // GROUP)
    bn, bk, sk = weight_geometry(N, K, w_s)
    out = np.empty(ms.shape, dtype=np.float64)
    _load().oracle_gemm_ref_at_geom(_p(a), _p(a_s), _p(w), _p(w_s), _p(ms), _p(ns),
                                    _p(out), ms.size, K, bn, bk, sk)
    return out


def gemm_bf16_ref(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """fp64 reference of the bf16 comparator GEMM, x[M,K] . w[N,K]^T: the bf16
    values are exact in fp64, and the product is numpy's float64 matmul (a
    library primitive as the one step; the pages' bf16 projection computes
    act . W^T, dispatch_proj.rs)."""
    xf = (np.ascontiguousarray(x_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    wf = (np.ascontiguousarray(w_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return xf.astype(np.float64) @ wf.astype(np.float64).T


# ------------------------------------------------------------------- FFN
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Values of bf16 bit patterns (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float64 values, one rounding to nearest even."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_f64_to_bf16_array(_p(v), _p(out), v.size)
    return out


def silu_mul(g_bits: np.ndarray, u_bits: np.ndarray):
    """h = bf16(silu(g) * u) of bf16 gate/up outputs, and the mask of the
    elements a binary32 evaluation may round to the other bf16 neighbour
    (see ``oracle_silu_mul``)."""
    g = np.ascontiguousarray(g_bits, dtype=np.uint16)
    u = np.ascontiguousarray(u_bits, dtype=np.uint16)
    assert g.shape == u.shape
    h = np.empty(g.shape, dtype=np.uint16)
    amb = np.empty(g.shape, dtype=np.uint8)
    _load().oracle_silu_mul(_p(g), _p(u), _p(h), _p(amb), g.size)
    return h, amb.astype(bool)


def ffn_ref(x_bits, wg, wg_s, wu, wu_s, wd, wd_s, rows=None) -> dict:
    """The dense FFN on FP8 weights, stage by stage (dispatch_proj.rs, doc of
    cublas_fp8_proj_prequant): the bf16 input x[M,H] is quantized once and
    feeds both the gate and the up projection (weights [I,H]); each
    projection's output is bf16 (the projection's output format); the
    intermediate h = bf16(silu(gate) * up) [M,I] is quantized once and feeds
    the down projection (weights [H,I]), whose fp64 result ``out`` [M,H] is
    left unrounded.

    ``rows`` restricts the chain to those token rows (every stage is
    row-local), for sampled checks at large M.  Returns the stages as a dict:
    xq, xs (x codes and row-major scales), g, u, h (bf16 bits), amb (the
    ``silu_mul`` mask), hq, hs (intermediate codes and row-major scales) and
    out."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if rows is not None:
        x = np.ascontiguousarray(x[np.asarray(rows, dtype=np.int64)])
    xq, xs = quant_act(x)
    g = f64_to_bf16(gemm_ref(xq, xs, wg, wg_s))
    u = f64_to_bf16(gemm_ref(xq, xs, wu, wu_s))
    h, amb = silu_mul(g, u)
    hq, hs = quant_act(h)
    out = gemm_ref(hq, hs, wd, wd_s)
    return dict(xq=xq, xs=xs, g=g, u=u, h=h, amb=amb, hq=hq, hs=hs, out=out)


# ---------------------------------------------------------------- tolerance
def bf16_ulp(r: np.ndarray) -> np.ndarray:
    """ulp of a bf16 number of magnitude |r|: 2^(max(floor(log2|r|), -126) - 7),
    and 2^-133 (the smallest bf16 subnormal) for r == 0."""
    r = np.abs(np.asarray(r, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    e = np.maximum(e, -126.0)
    u = np.ldexp(1.0, (e - 7).astype(np.int64))
    return np.where(r > 0, u, np.ldexp(1.0, -133))


def round_to_bf16(r: np.ndarray) -> np.ndarray:
    """The fp64 reference in the output format: each value rounded once, to
    nearest with ties to even, to a bf16 value (returned as float64).  r/ulp is
    an exact power-of-two rescaling, and numpy's rint rounds half to even."""
    r = np.asarray(r, dtype=np.float64)
    u = bf16_ulp(r)
    return np.rint(r / u) * u


def gemm_errors(out_bf16_as_f64: np.ndarray, ref: np.ndarray, rms_ref: float | None = None):
    """Accuracy of a bf16 GEMM output against the oracle's fp64 product.

    Returns (rel_rms, excess, rel_rms_f64):
      rel_rms      sqrt(sum (o - b)^2 / sum b^2), b = round_to_bf16(ref): the
                   relative RMS error against the reference in the output's
                   format (the rounding of any bf16 output to the fp64 value
                   alone costs a relative RMS of ~1.66e-3, so the 1e-3 bar is
                   taken against the bf16-rounded reference)
      excess       max |o - r| / (ulp_bf16(r) + 1e-3 * RMS(ref)) against the
                   unrounded fp64 reference r; the bar is excess <= 1
      rel_rms_f64  the relative RMS error against the unrounded reference
                   (information: about 1.66e-3 for any bf16 output)
    ``rms_ref`` overrides RMS(ref) (for sampled comparisons)."""
    o = np.asarray(out_bf16_as_f64, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if rms_ref is None:
        rms_ref = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    b = round_to_bf16(r)

    def rel(x, y):
        d = x - y
        den = float(np.sum(y * y))
        return float(np.sqrt(np.sum(d * d) / den)) if den > 0 else float(np.sqrt(np.sum(d * d)))

    bound = bf16_ulp(r) + 1e-3 * rms_ref
    excess = float(np.max(np.abs(o - r) / bound)) if r.size else 0.0
    return rel(o, b), excess, rel(o, r)
