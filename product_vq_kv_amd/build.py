"""Compile the HIP library libvq.so for gfx950, in-tree.

    python product_vq_kv_amd/build.py     (a script: it imports nothing of the package)

Flags:
  * --offload-arch=gfx950: CDNA4 only, no other targets;
  * -Xclang -target-feature -Xclang -packed-fp32-ops: no packed-fp32 VALU
    instructions are generated;
  * -ffp-contract=off: the only fused operations are the explicit fmaf calls,
    so the distance arithmetic is exactly the documented sequence;
  * -fno-gpu-flush-denormals-to-zero: fp32 subnormals are kept, as IEEE (and
    the CPU reference) does;
  * -mllvm -amdgpu-mfma-vgpr-form: matrix-core results land in ordinary VGPRs,
    so the VALU reduction reads them without v_accvgpr_read copies.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libvq.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources() -> list[str]:
    csrc = os.path.join(HERE, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.cpp")))


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str = LIB) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []),
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           *sources(), "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
