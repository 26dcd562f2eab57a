"""Build libgqa_attn.so (HIP kernels + host planner + C ABI) for gfx950.

Usage: python -m gqa_attention_agentic_amd.build [--verbose] [--resource-usage]

The library is built in-tree next to this file. Every HIP translation unit is
compiled with packed-fp32 instructions disabled (the compiler otherwise emits
v_pk_* fp32 ops from ordinary float code).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgqa_attn.so")
ARCH = "gfx950"

SOURCES = ["attention.hip", "append.hip", "fill.hip", "scratch.hip", "probe.hip", "api.cpp", "plan.cpp"]
NO_PACKED_FP32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Kernels run with the IEEE mode bit off: max/min then need no NaN-quieting
# canonicalisation of their inputs. The kernels never produce NaN themselves
# (masked scores are -inf and the -inf - -inf case is guarded).
KERNEL_FP = ["-mno-amdgpu-ieee", "-fno-honor-nans"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP extension)")


def build(verbose: bool = False, resource_usage: bool = False, defines=(), lib_path: str = LIB) -> str:
    cc = hipcc()
    objs = []
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
              f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(bdir, src + ("." + "_".join(defines) if defines else "") + ".o")
        cmd = [cc] + common + NO_PACKED_FP32 + [f"-D{d}" for d in defines]
        if src.endswith(".hip"):
            cmd += KERNEL_FP
        if src.endswith(".hip") and resource_usage:
            cmd += ["-Rpass-analysis=kernel-resource-usage"]
        cmd += ["-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in line)
        if r.returncode != 0:
            raise RuntimeError(f"compile of {src} failed:\n{out}")
        if out.strip() and (verbose or resource_usage):
            print(out, flush=True)
        objs.append(obj)
    tmp = lib_path + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, resource_usage="--resource-usage" in sys.argv))
