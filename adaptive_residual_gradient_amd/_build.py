"""Build of the HIP library ``libadacomp.so`` for gfx950 with hipcc."""
from __future__ import annotations

import os
import pathlib
import subprocess

HERE = pathlib.Path(__file__).resolve().parent
SRC = HERE / "csrc" / "adacomp.hip"
LIB = HERE / "libadacomp.so"

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Bit-exact float32: no contraction of a*b+c into fused multiply-adds.
    "-ffp-contract=off",
    # No packed fp32 instructions (v_pk_add_f32 and friends).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> pathlib.Path:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc, *HIPCC_FLAGS, "-o", str(tmp), str(SRC)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
