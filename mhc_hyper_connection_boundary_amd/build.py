"""Builds libmhc.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each source compiles to its own object in parallel (each object carries its
own gfx950 code object; no relocatable device code is needed, since no kernel
calls device code in another file), then one hipcc call links the library.
"""
from __future__ import annotations

import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmhc.so")
SOURCES = ["mhc_api.hip", "mhc_kernels.hip", "mhc_fused.hip", "mhc_stream.hip", "mhc_pre_one.hip"]
# The LDS-poison debug build: the same sources with -DMHC_LDS_POISON (every
# kernel fills its LDS with NaN before use); the tests run it beside libmhc.so.
POISON_LIB = os.path.join(PKG, "libmhc_lds_poison.so")
# The movers (a measurement tool for bench.py; mhc_boundary never calls them).
MOVER_LIB = os.path.join(PKG, "libmhc_mover.so")
MOVER_SOURCE = "mhc_mover.hip"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Further compilations of a source, each with its own defines and flags: the
# fused boundary kernels at hidden 7168 under other LLVM machine schedulers
# (mhc_fused.hip holds the measurements).
EXTRA_UNITS = [("mhc_fused.hip", "mhc_fused_maxilp",
                ["-DMHC_FUSED_MAXILP", "-mllvm", "-amdgpu-sched-strategy=max-ilp"]),
               ("mhc_fused.hip", "mhc_fused_maxclause",
                ["-DMHC_FUSED_MAXCLAUSE", "-mllvm", "-amdgpu-sched-strategy=max-memory-clause"])]

ARCH = ["--offload-arch=gfx950"]
FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    # packed FP32 instructions stay off (v_pk_fma_f32 and friends are not used)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd: list[str], verbose: bool) -> str:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{msgs}")
    return msgs


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="mhc_build_") as tmp:
        units = [(s, os.path.splitext(s)[0], []) for s in SOURCES] + EXTRA_UNITS
        jobs = []
        for s, name, extra in units:
            obj = os.path.join(tmp, name + ".o")
            cmd = [HIPCC, *ARCH, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"),
                   "-c", os.path.join(CSRC, s), "-o", obj]
            if resource_usage:
                cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
            jobs.append((cmd, obj))
        poison_jobs = []
        for s, name, extra in units:
            obj = os.path.join(tmp, "poison_" + name + ".o")
            poison_jobs.append(([HIPCC, *ARCH, *FLAGS, *extra, "-DMHC_LDS_POISON", "-I", os.path.join(ROOT, "include"),
                                 "-c", os.path.join(CSRC, s), "-o", obj], obj))
        mover_obj = os.path.join(tmp, "mhc_mover.o")
        mover_cmd = [HIPCC, *ARCH, *FLAGS, "-c", os.path.join(CSRC, MOVER_SOURCE), "-o", mover_obj]
        with ThreadPoolExecutor(max_workers=min(16, 2 * len(jobs) + 1)) as ex:
            outs = list(ex.map(lambda j: _run(j[0], verbose), jobs + poison_jobs + [(mover_cmd, mover_obj)]))
        outs.append(_run([HIPCC, *ARCH, "-shared", "-fPIC", *(o for _, o in jobs),
                          "-o", LIB + ".tmp"], verbose))
        if verbose:
            for m in outs:
                if m.strip():
                    print(m)
        os.replace(LIB + ".tmp", LIB)
        outs.append(_run([HIPCC, *ARCH, "-shared", "-fPIC", mover_obj, "-o", MOVER_LIB + ".tmp"], verbose))
        os.replace(MOVER_LIB + ".tmp", MOVER_LIB)
        outs.append(_run([HIPCC, *ARCH, "-shared", "-fPIC", *(o for _, o in poison_jobs),
                          "-o", POISON_LIB + ".tmp"], verbose))
        os.replace(POISON_LIB + ".tmp", POISON_LIB)
    return LIB


if __name__ == "__main__":
    import sys
    build(verbose=True, resource_usage="--resources" in sys.argv)
