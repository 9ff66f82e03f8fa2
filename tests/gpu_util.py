"""Helpers for the GPU parity tests: device transfers and canary-guarded
output buffers.  Imported only by tests marked ``gpu``."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth

CANARY = 0xA5  # byte pattern written after every output buffer
PAD_BYTES = 4096


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> contiguous GPU tensor of the same bytes (uint16 -> int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(a)
    return t.cuda()


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


class Guarded:
    """An output tensor of `shape`/`dtype` followed by PAD_BYTES of canary, and
    preceded by PAD_BYTES of canary (16-byte aligned view in the middle)."""

    def __init__(self, shape, dtype, fill: int = 0x5A):
        self.shape = tuple(shape)
        self.dtype = dtype
        esize = torch.empty((), dtype=dtype).element_size()
        self.nbytes = int(np.prod(self.shape)) * esize
        self.raw = torch.full((self.nbytes + 2 * PAD_BYTES,), CANARY, dtype=torch.uint8,
                              device="cuda")
        self.raw[PAD_BYTES:PAD_BYTES + self.nbytes] = fill
        self.t = self.raw[PAD_BYTES:PAD_BYTES + self.nbytes].view(dtype).view(self.shape)

    def check_canary(self):
        r = self.raw.cpu().numpy()
        assert np.all(r[:PAD_BYTES] == CANARY), "write before the start of an output buffer"
        assert np.all(r[PAD_BYTES + self.nbytes:] == CANARY), "write past the end of an output buffer"


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(a.view(np.uint16)).astype(np.float64)


def require_gpu():
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), f"expected gfx950, got {name}"


RTOL = 1e-3  # relative-RMS bar of the GEMM outputs


def assert_tol(o, r, what, rms=None):
    """The GEMM accuracy contract against the oracle's fp64 product r:
    rel_rms <= RTOL against r rounded to bf16 (the output format) and, for
    every element, |o - r| <= ulp_bf16(r) + 1e-3 * RMS(r).  rms: RMS(r) when
    r is a sample of the output (else it is taken from r)."""
    import oracle
    rel, exc, relf = oracle.gemm_errors(o, r, rms)
    log(f"  {what}: rel_rms={rel:.3e} (vs fp64 {relf:.3e}) worst/bound={exc:.3f}")
    assert rel <= RTOL, f"{what}: rel_rms {rel}"
    assert exc <= 1.0, f"{what}: per-element error {exc} x bound"
