"""Build librec.so (the HIP library) in-tree for gfx950.

    python -m sparse_embedding_din_amd.build

Every HIP source is compiled with -packed-fp32-ops disabled (no packed fp32
instructions are generated) and with matrix-core results kept in ordinary
VGPRs where they fit (-amdgpu-mfma-vgpr-form): the attention's epilogues read
every accumulator, and reading them from AGPRs costs a copy per value."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "librec.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-Wall", "-I", os.path.join(ROOT, "include"), "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in l]
    if r.returncode != 0:
        raise RuntimeError("librec build failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    sys.exit(0)
