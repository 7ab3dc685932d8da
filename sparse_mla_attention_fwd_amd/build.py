"""Build libsmla.so (gfx950 kernels + C-ABI layer) in-tree with hipcc.

Run as ``python -m sparse_mla_attention_fwd_amd.build`` (``--poison``: the
LDS-poisoning debug library, ``--all``: both) or call ``build()`` /
``build_all()``.  The shared libraries land next to this file, where the
binding loads them.
"""
from __future__ import annotations

import os
import shutil
from concurrent.futures import ThreadPoolExecutor
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsmla.so")
# LDS-poisoning debug build (tests only; see build())
POISON_LIB = os.path.join(HERE, "libsmla_poison.so")
# The forward kernels are split over several translation units (one per group
# of launch configurations) so that they compile in parallel.
SOURCES = ["smla_fwd_bf16_persist.hip", "smla_fwd_bf16_b128.hip", "smla_fwd_fp8_w4.hip", "smla_fwd_fp8_w1w2.hip", "smla_fwd_fp4.hip", "smla_fwd_bf16_w4_b32.hip",
           "smla_fwd_bf16_w4_b64.hip", "smla_fwd_bf16_w1.hip", "smla_fwd_bf16_w2.hip",
           "smla_launch.hip", "smla_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False, poison: bool = False) -> str:
    """Compile every source for gfx950 and link libsmla.so; returns its path.

    poison=True builds the LDS-poisoning debug library libsmla_poison.so
    instead (SMLA_DEBUG_LDS_POISON: every kernel fills its LDS with NaN bytes
    at entry and before each direct-to-LDS load, so that races and reads of
    unwritten LDS surface as NaN in the results)."""
    return build_variants(verbose, (poison,))[0]


def build_all(verbose: bool = False) -> tuple[str, str]:
    """The product library and the LDS-poisoning debug library, compiled in one
    pool; returns both paths."""
    lib, dbg = build_variants(verbose, (False, True))
    return lib, dbg


def compile_flags(poison: bool = False) -> list[str]:
    """hipcc flags of every translation unit (poison: the debug build)."""
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        # packed fp32 VALU ops are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ] + (["-DSMLA_DEBUG_LDS_POISON=1"] if poison else [])


def build_variants(verbose: bool, variants: tuple[bool, ...]) -> list[str]:
    cc = hipcc()

    def objdir(poison: bool) -> str:
        d = os.path.join(HERE, "_build_poison" if poison else "_build")
        os.makedirs(d, exist_ok=True)
        return d

    def compile_one(job: tuple[bool, str]) -> str:
        poison, src = job
        obj = os.path.join(objdir(poison), src + ".o")
        cmd = [cc, *compile_flags(poison), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    jobs_list = [(v, src) for v in variants for src in SOURCES]
    jobs = max(1, min(len(jobs_list), os.cpu_count() or 1, int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, jobs_list))
    out = []
    for i, poison in enumerate(variants):
        lib = POISON_LIB if poison else LIB
        tmp = lib + ".tmp"
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs[i * len(SOURCES):(i + 1) * len(SOURCES)],
               "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp, lib)
        out.append(lib)
    return out


if __name__ == "__main__":
    if "--poison" in sys.argv:
        print(build(verbose="-v" in sys.argv, poison=True))
    elif "--all" in sys.argv:
        print(*build_all(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
