"""Build the measurement programs of this folder for gfx950.

    python bench/micro/build.py        # -> bench/micro/gather_ceiling, issue_probe, lds_patterns

They are standalone HIP programs (they allocate their own buffers) that
measure the hardware limits behind the forward kernels' design: the random-row
gather ceiling of the memory system, the issue rate of one wave's MFMAs and the
LDS cost of the operand-read patterns of two stage layouts.
They are not part of the library and are not built with it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PROGRAMS = ("gather_ceiling", "issue_probe", "lds_patterns")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(name: str, verbose: bool = False) -> str:
    exe = os.path.join(HERE, name)
    cmd = [hipcc(), "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-x", "hip", os.path.join(HERE, name + ".cpp"), "-o", exe + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {name}.cpp:\n{r.stderr}")
    os.replace(exe + ".tmp", exe)
    return exe


if __name__ == "__main__":
    for n in PROGRAMS:
        print(build(n, verbose="-v" in sys.argv))
