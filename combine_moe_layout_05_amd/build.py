"""Build libmoe_layout.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python combine_moe_layout_05_amd/build.py
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

if __package__:
    from ._paths import LIB_PATH, PKG, PROBE_LIB_PATH
else:  # run as a script
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from _paths import LIB_PATH, PKG, PROBE_LIB_PATH  # type: ignore

ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")

SOURCES = ["layout.hip", "dispatch.hip", "combine.hip", "combine_backward.hip", "routing_map.hip",
           "grouped_gemm.hip", "noalloc.hip",
           "moe_api.cpp"]
HEADERS = [os.path.join(CSRC, "moe_kernels.h"), os.path.join(CSRC, "moe_lanes.h"),
           os.path.join(INCLUDE, "moe.h")]
# The benchmark's traffic reference kernels, built into a library of their own.
PROBE_SOURCES = ["traffic_probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Packed fp32 vector ops stay off; the kernels never rely on them.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Every multiply-add in the combine is an explicit fmaf; nothing else
    # is contracted, and fp32 denormals are kept (IEEE).
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    # Kernel arguments preloaded into SGPRs when a wavefront starts (gfx950),
    # instead of each wavefront's first scalar load of them. Measured on
    # MI355X, per step, four interleaved runs of 200 steps: 180.6-180.7
    # against 181.0-181.3 us at 4096 tokens of 7168, 212.3-212.5 against
    # 213.0-213.6 us at 8192 tokens of 4096, 32.3-32.4 against 32.7 us at
    # 2047 tokens of 2048 (the layout gains most, 0.3-0.6 us).
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    """Compile every source into combine_moe_layout_05_amd/libmoe_layout.so
    (one hipcc process per source file in parallel, then one link), and the
    benchmark's traffic reference kernels into libmoe_traffic_probe.so."""
    lib = _build_library(SOURCES, LIB_PATH, verbose)
    _build_library(PROBE_SOURCES, PROBE_LIB_PATH, verbose)
    return lib


def _build_library(sources, out_path: str, verbose: bool) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    procs = []
    objs = []
    for src in sources:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        cmd = [hipcc(), *compile_flags, "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(out)
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc link failed with status {res.returncode}")
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
