"""Build libfp8q.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m w8a8_fp8_block_amd.build

hipcc cross-compiles for gfx950 without a GPU present.  Flags:
  -O3 --offload-arch=gfx950           the only target
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                      keep the compiler from emitting packed
                                      fp32 VALU ops (the host pass warns that
                                      it does not know the feature: harmless)
  -mllvm -amdgpu-mfma-vgpr-form       MFMA results in VGPRs: every GEMM partial
                                      product is consumed by VALU fmas, which
                                      cannot read AGPRs
  -fgpu-flush-denormals-to-zero is NOT given: the quantizer relies on IEEE
  subnormal fp32 arithmetic (the default).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libfp8q.so")
SOURCES = ["fp8q_api.hip", "quant.hip", "relayout.hip", "gemm.hip", "gemm_bf16.hip", "dequant.hip",
           "ffn.hip", "clock.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
