"""Brute-force reference for tiny inputs -- an implementation of the
activation quantizer that shares nothing with the oracle's C code.

* The e4m3 value table comes from PyTorch's ``float8_e4m3fn`` dtype (a library
  routine), not from a formula.
* Encoding is a search: the finite table value nearest to q, ties broken
  toward the code with an even mantissa (even low bit), magnitudes at or above
  the largest finite value saturate to it.
* fp32 quotients are computed in binary64 and rounded once to binary32 by
  numpy.  A quotient of two 24-bit numbers computed with 53 >= 2*24 + 2 bits
  and then rounded to 24 bits equals the correctly rounded quotient (double
  rounding is innocuous at that precision), so this is IEEE fp32 division.

Pure Python loops; use only on a few thousand elements.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def _value_table():
    codes = torch.arange(256, dtype=torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float64).tolist()
    return vals


VALUES = _value_table()
# positive finite codes, by value
_POS = sorted((v, c) for c, v in enumerate(VALUES) if c < 0x80 and not math.isnan(v))
MAXV = _POS[-1][0]


def f32(v: float) -> float:
    return float(np.float32(v))


def bf16_value(bits: int) -> float:
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def encode(q: float) -> int:
    """Nearest e4m3fn code by exhaustive search (ties -> even mantissa)."""
    neg = math.copysign(1.0, q) < 0
    a = abs(q)
    if a >= MAXV:
        best = _POS[-1][1]
    else:
        best, bestd = None, None
        for v, c in _POS:
            d = abs(v - a)
            if bestd is None or d < bestd or (d == bestd and (c & 1) == 0):
                best, bestd = c, d
    return best | (0x80 if neg else 0)


def quant_act(x_bits: np.ndarray):
    """bf16 bits [M,K] -> (codes [M,K] uint8, scales [M,K/128] float32)."""
    M, K = x_bits.shape
    G = K // 128
    codes = np.zeros((M, K), dtype=np.uint8)
    scales = np.zeros((M, G), dtype=np.float32)
    for m in range(M):
        for g in range(G):
            xs = [bf16_value(int(b)) for b in x_bits[m, 128 * g:128 * (g + 1)]]
            amax = max(abs(v) for v in xs)
            s = f32(amax / 448.0)
            scales[m, g] = s
            for j, v in enumerate(xs):
                if s == 0.0:
                    c = 0x80 if math.copysign(1.0, v) < 0 else 0x00
                else:
                    c = encode(f32(v / s))
                codes[m, 128 * g + j] = c
    return codes, scales


def kmajor(scales_rm: np.ndarray) -> np.ndarray:
    """Relayout by explicit index loops: km[g][m] for m < ceil16(M)."""
    M, G = scales_rm.shape
    Mp = -(-M // 16) * 16
    km = np.full((G, Mp), np.nan, dtype=np.float32)
    for g in range(G):
        for m in range(Mp):
            km[g, m] = scales_rm[m, g] if m < M else 0.0
    return km
