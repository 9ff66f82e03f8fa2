"""Seeded synthetic inputs for the W8A8 block-scaled FP8 projection.

This module is the only code shared by the oracle tests, the GPU parity tests
and the benchmark.  It draws random numbers and lays out bit patterns; it does
none of the method's arithmetic (no quantization, no scaling, no GEMM).

Inputs follow the shapes of the projection workloads:

* activations: bf16 ``[M, K]`` drawn from N(0, 1) (or Laplace(0, 1)), with a
  few "outlier" channels (whole K columns) multiplied by a constant factor;
* weights: fp32 ``[N, K]`` drawn from N(0, 0.02), to be block-quantized to FP8
  by whoever consumes them.

Draw order is fixed so a (workload, seed) pair always yields the same bytes:
outlier channel indices, then activations, then weights, all from one
``numpy.random.default_rng(seed)`` (PCG64).
"""
from __future__ import annotations

import dataclasses
from typing import Iterator

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_inputs",
    "ceil16",
    "exhaustive_pair_groups",
    "n_exhaustive_groups",
    "FfnWorkload",
    "FFN_WORKLOADS",
    "ffn_workload",
    "make_ffn_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int  # 0 for the quantizer-only sweep
    dist: str  # "normal" or "laplace"
    n_outliers: int
    outlier_factor: float
    seed: int = 0

    @property
    def desc(self) -> str:
        return f"{self.name}:M{self.M}xK{self.K}xN{self.N}"


def _n_out(frac: float, K: int) -> int:
    return int(round(frac * K))


def _mk(name, M, K, N, dist, n_out, factor) -> Workload:
    return Workload(name, M, K, N, dist, n_out, factor, 0)


# The five synthetic projection workloads (sizes of real model projections).
WORKLOADS: dict[str, list[Workload]] = {
    # tiny: M=16, K=512, N=256, 2 outlier channels x20
    "tiny": [_mk("tiny", 16, 512, 256, "normal", 2, 20.0)],
    # decode-width sweep: M in {16,17,25}, K=5120, N=6144, 1% outliers x20
    "decode": [_mk("decode", m, 5120, 6144, "normal", _n_out(0.01, 5120), 20.0)
               for m in (16, 17, 25)],
    # prefill gate/up-like: M=1168, K=5120, N=17408
    "prefill": [_mk("prefill", 1168, 5120, 17408, "normal", _n_out(0.01, 5120), 20.0)],
    # large prefill down-proj-like: Laplace acts, 0.5% outliers x50
    "large_prefill": [_mk("large_prefill", 4576, 17408, 5120, "laplace",
                          _n_out(0.005, 17408), 50.0)],
    # quantizer + relayout only
    "quant_sweep": [_mk("quant_sweep", m, k, 0, "normal", _n_out(0.01, k), 20.0)
                    for m in (16, 25, 1168, 4576, 16384) for k in (5120, 6144, 17408)],
}


def workload(name: str, M: int | None = None, K: int | None = None) -> Workload:
    """Look up one workload by name (and M/K for the sweeps)."""
    for w in WORKLOADS[name]:
        if (M is None or w.M == M) and (K is None or w.K == K):
            return w
    raise KeyError((name, M, K))


def ceil16(m: int) -> int:
    return (m + 15) // 16 * 16


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_inputs(w: Workload, M: int | None = None, with_weights: bool = True,
                seed: int | None = None):
    """Draw (x_bf16 [M,K] uint16, w_f32 [N,K] float32 or None, outlier idx).

    ``M`` overrides the workload's row count (used for smaller parity runs of
    the same K/N); ``seed`` overrides its seed.
    """
    M = w.M if M is None else M
    rng = np.random.default_rng(w.seed if seed is None else seed)
    out_idx = rng.choice(w.K, w.n_outliers, replace=False) if w.n_outliers else \
        np.zeros(0, dtype=np.int64)
    if w.dist == "normal":
        x = rng.standard_normal((M, w.K), dtype=np.float32)
    elif w.dist == "laplace":
        x = rng.laplace(0.0, 1.0, (M, w.K)).astype(np.float32)
    else:
        raise ValueError(w.dist)
    if len(out_idx):
        x[:, out_idx] *= np.float32(w.outlier_factor)
    xb = f32_to_bf16_bits(x)
    del x
    wf = None
    if with_weights and w.N:
        wf = rng.normal(0.0, 0.02, (w.N, w.K)).astype(np.float32)
    return xb, wf, out_idx


# --------------------------------------------------------------------------
# Dense FFN chain: x [M,H] -> gate, up [I,H] -> SiLU(gate) * up -> down [H,I].
# Sizes of the projections above: gate/up are the prefill shape (K=5120,
# N=17408 each) and down the large-prefill shape (K=17408, N=5120).
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class FfnWorkload:
    name: str
    M: int
    H: int  # model width: x and out are [M,H]
    I: int  # intermediate width: gate/up are [I,H], down is [H,I]
    n_outliers: int
    outlier_factor: float
    seed: int = 0

    @property
    def desc(self) -> str:
        return f"{self.name}:M{self.M}xH{self.H}xI{self.I}"


FFN_WORKLOADS: dict[str, list[FfnWorkload]] = {
    "ffn_tiny": [FfnWorkload("ffn_tiny", 16, 256, 384, 2, 20.0)],
    "ffn_decode": [FfnWorkload("ffn_decode", m, 5120, 17408, _n_out(0.01, 5120), 20.0)
                   for m in (16, 25)],
    "ffn_prefill": [FfnWorkload("ffn_prefill", 1168, 5120, 17408, _n_out(0.01, 5120), 20.0)],
    "ffn_large": [FfnWorkload("ffn_large", 4576, 5120, 17408, _n_out(0.01, 5120), 20.0)],
}


def ffn_workload(name: str, M: int | None = None) -> FfnWorkload:
    for w in FFN_WORKLOADS[name]:
        if M is None or w.M == M:
            return w
    raise KeyError((name, M))


def make_ffn_inputs(w: FfnWorkload, M: int | None = None, seed: int | None = None,
                    with_weights: bool = True):
    """Draw (x_bf16 [M,H] uint16, (w_gate [I,H], w_up [I,H], w_down [H,I])
    float32 or None).  Activations: N(0,1) with outlier channels; weights:
    N(0, 0.02), to be block-quantized to FP8 by whoever consumes them.  Draw
    order: outlier indices, x, gate, up, down."""
    M = w.M if M is None else M
    rng = np.random.default_rng(w.seed if seed is None else seed)
    out_idx = rng.choice(w.H, w.n_outliers, replace=False) if w.n_outliers else \
        np.zeros(0, dtype=np.int64)
    x = rng.standard_normal((M, w.H), dtype=np.float32)
    if len(out_idx):
        x[:, out_idx] *= np.float32(w.outlier_factor)
    xb = f32_to_bf16_bits(x)
    del x
    if not with_weights:
        return xb, None
    wg = rng.normal(0.0, 0.02, (w.I, w.H)).astype(np.float32)
    wu = rng.normal(0.0, 0.02, (w.I, w.H)).astype(np.float32)
    wd = rng.normal(0.0, 0.02, (w.H, w.I)).astype(np.float32)
    return xb, (wg, wu, wd)


# --------------------------------------------------------------------------
# Exhaustive (x, amax) enumeration.  Inside one 128-wide group the FP8 code of
# an element depends only on the element and the group's absolute maximum, so
# every finite positive bf16 amax paired with every bf16 x, |x| <= amax, covers
# the whole element map.  Each group holds its amax once followed by 127 test
# values.
# --------------------------------------------------------------------------
_MAX_FINITE_BF16 = 0x7F7F


def _pairs_per_amax(a: int) -> int:
    # test values 0..a (bit patterns), both signs (+0 and -0 both included)
    return 2 * (a + 1)


def n_exhaustive_groups(amax_lo: int = 1, amax_hi: int = _MAX_FINITE_BF16) -> int:
    a = np.arange(amax_lo, amax_hi + 1, dtype=np.int64)
    return int(np.sum((_pairs_per_amax(a) + 126) // 127))


def exhaustive_pair_groups(amax_lo: int, amax_hi: int) -> np.ndarray:
    """Groups (rows of 128 bf16 bit patterns) covering every (x, amax) pair
    with amax in the bit-pattern range [amax_lo, amax_hi] (positive, finite).

    Column 0 of each row is amax; columns 1..127 hold x values (bit patterns
    0..amax with sign bit clear, then with sign bit set, -0.0 included);
    unused slots of a row's tail repeat +0, which never changes the group
    maximum.
    """
    rows = []
    for a in range(amax_lo, amax_hi + 1):
        mags = np.arange(0, a + 1, dtype=np.uint16)
        vals = np.concatenate([mags, mags | np.uint16(0x8000)])
        ng = (len(vals) + 126) // 127
        buf = np.zeros(ng * 127, dtype=np.uint16)
        buf[: len(vals)] = vals
        g = np.empty((ng, 128), dtype=np.uint16)
        g[:, 0] = a
        g[:, 1:] = buf.reshape(ng, 127)
        rows.append(g)
    return np.concatenate(rows, axis=0)


def exhaustive_chunks(max_groups: int) -> Iterator[tuple[int, int]]:
    """Split the positive finite bf16 amax range into chunks of at most about
    ``max_groups`` groups each; yields (amax_lo, amax_hi) pairs."""
    lo = 1
    acc = 0
    for a in range(1, _MAX_FINITE_BF16 + 1):
        acc += (_pairs_per_amax(a) + 126) // 127
        if acc >= max_groups:
            yield lo, a
            lo, acc = a + 1, 0
    if lo <= _MAX_FINITE_BF16:
        yield lo, _MAX_FINITE_BF16
