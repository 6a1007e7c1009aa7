"""Build libupipe_attn.so in-tree with hipcc for gfx950.

    python -m headwise_chunked_context_amd.build [--verbose]

Compiles every csrc/*.hip to an object (in parallel) and links one shared
library next to this file.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libupipe_attn.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-munsafe-fp-atomics",
    # packed fp32 VALU ops stay off (v_pk_*_f32); plain scalar float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # device code never relies on NaN semantics (masked scores are -inf, not
    # NaN); this lets fmaxf lower to v_max/v_max3 without quieting its inputs
    "-Xarch_device", "-fno-honor-nans",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


# Per-file additions (none at present).  The dQ kernel's file once took
# LLVM's max-ILP machine scheduler (-mllvm -amdgpu-sched-strategy=max-ilp),
# 2.5% faster for the kernel of that time; with its score chains started
# from the -LSE tuple the default strategy is 0.5% faster, and the dK/dV
# kernel always measured 3% slower with max-ILP.
FILE_FLAGS: dict[str, list[str]] = {}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJ, exist_ok=True)
    flags = HIPCC_FLAGS + list(extra_flags or [])

    def compile_one(src: str) -> str:
        obj = os.path.join(OBJ, os.path.basename(src).replace(".hip", ".o"))
        cmd = [hipcc, *flags, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        out = (res.stdout + res.stderr).strip()
        # the host pass does not know the packed-fp32 feature name; harmless
        noise = "'-packed-fp32-ops' is not a recognized feature"
        out = "\n".join(l for l in out.splitlines() if noise not in l)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{out}")
        if verbose and out:
            print(out)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, sources()))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
