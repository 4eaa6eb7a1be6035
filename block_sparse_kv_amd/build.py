"""Builds libmage.so (the gfx950 HIP library behind include/mage.h) in-tree.

    python -m block_sparse_kv_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmage.so")
SOURCES = [os.path.join(PKG, "csrc", "mage_api.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # keep packed-fp32 VALU instructions (v_pk_fma_f32 and kin) out of the code
    # object: the kernels are written and checked for scalar fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in architectural VGPRs: the later step, score sweep and block
    # attention otherwise keep their accumulators in AGPRs and copy them to VGPRs
    # for every rescale and read (272 copies in the later step's loop at d=128)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def build(extra_flags=(), out: str = LIB) -> str:
    """Compile every HIP source for gfx950 into `out` (always recompiles)."""
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra_flags, "-o", tmp, *SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
