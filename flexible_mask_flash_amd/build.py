"""Build libffa.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m flexible_mask_flash_amd.build [--asm]

--asm also writes the device assembly next to the library (for inspection of
register use, waitcnt placement and MFMA scheduling).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libffa.so")
ARCH = "gfx950"

SOURCES = ["ffa_plan.cpp", "ffa_fwd.hip", "ffa_bwd.hip", "ffa_bwd_small.hip"]

# Packed fp32 VALU ops are disabled: the compiler must not form v_pk_{add,mul,fma}_f32.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-honor-nans"]
# Per-source device flags.  The backward's score products feed VALU work (exp2,
# dS) directly, so their MFMAs must write arch VGPRs: left to its heuristic, the
# compiler gives every MFMA of a one-wave-per-SIMD kernel an AGPR destination and
# then copies each score out and back (v_accvgpr_read / write around every exp2).
# The backward's D >= 64 kernels also take the max-ILP machine scheduler: the same
# instructions and results (bitwise), +0.2 to +1.9% on the D >= 64 backward workloads in
# same-process A/B runs; at D = 32 and 16 it measured -3%, so those instances are compiled
# in ffa_bwd_small.hip under the default scheduler.  The forward measured slower with it
# (-0.1 to -1.1%) and keeps the default.
_BWD_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
SOURCE_FLAGS = {
    "ffa_bwd.hip": _BWD_FLAGS + ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "ffa_bwd_small.hip": _BWD_FLAGS,
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libffa.so)")


def asm_command(src: str, out_path: str) -> list:
    """hipcc command writing the gfx950 device assembly of a .hip source, with the flags
    the library is built with."""
    common = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function"]
    return [hipcc(), *common, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "--cuda-device-only", "-S",
            os.path.join(CSRC, src), "-o", out_path]


def build(verbose: bool = False, asm: bool = False) -> str:
    """Compile every source and link libffa.so; returns the library path."""
    cc = hipcc()
    objs = []
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function"]
    jobs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(bdir, src + ".o")
        cmd = [cc, *common]
        if src.endswith(".hip"):
            cmd += DEVICE_FLAGS + SOURCE_FLAGS.get(src, [])
        else:
            cmd += ["-x", "c++"]
        cmd += ["-c", path, "-o", obj]
        jobs.append(cmd)
        objs.append(obj)
        if asm and src.endswith(".hip"):
            jobs.append(asm_command(src, os.path.join(bdir, src + f".{ARCH}.s")))
    # the sources compile independently
    with ThreadPoolExecutor(max_workers=min(len(jobs), 4)) as ex:
        for f in [ex.submit(_run, cmd, verbose) for cmd in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True, asm="--asm" in sys.argv))
