"""Build libe3hip.so (gfx950) in-tree.

Steps:
  1. compile and run the host CG generator (csrc/host) to write
     csrc/generated/cg_table.inc, the record table the kernels unroll;
  2. compile every HIP / C++ source with hipcc for gfx950;
  3. link clebsch_gordan_tensor_amd/libe3hip.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libe3hip.so")
ARCH = "gfx950"

HIP_SOURCES = [
    "kernels/inst_l1.hip",
    "kernels/inst_l1to3.hip",
    "kernels/inst_l2to3.hip",
    "kernels/inst_l3to3.hip",
    "kernels/inst_l1to3all.hip",
    "kernels/inst_per_path.hip",
    "kernels/prep.hip",
    "kernels/linear.hip",
    "kernels/radial.hip",
    "kernels/generic.hip",
    "kernels/gemm.hip",
    "api.cpp",
    "host/cg_ladder.cpp",
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions anywhere (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose, log=None):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # hipcc's host pass does not know the device feature: not an error
    out = "\n".join(l for l in out.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if log is not None:
        log.append(out)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("command failed: " + " ".join(cmd))
    if verbose and out.strip():
        print(out, flush=True)


def generate_tables(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(os.path.join(CSRC, "generated"), exist_ok=True)
    exe = os.path.join(BUILD, "gen_cg_table")
    _run(["g++", "-O2", "-std=c++17", "-Wall", "-o", exe,
          os.path.join(CSRC, "host", "gen_cg_table.cpp"),
          os.path.join(CSRC, "host", "cg_ladder.cpp")], verbose)
    out = os.path.join(CSRC, "generated", "cg_table.inc")
    _run([exe, out + ".tmp"], verbose)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False, resource_usage: bool = False, jobs: int | None = None) -> str:
    generate_tables(verbose)
    objs, logs = [], []
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
        log = []
        _run([HIPCC] + HIP_FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj], verbose,
             log)
        return obj, log

    jobs = jobs or min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        for obj, log in ex.map(compile_one, HIP_SOURCES):
            objs.append(obj)
            logs.extend(log)
    if resource_usage:
        with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
            f.write("\n".join(logs))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, resource_usage="--usage" in sys.argv))
