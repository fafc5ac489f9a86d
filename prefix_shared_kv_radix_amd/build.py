"""Build libradix_attn.so in-tree: host C++ with g++, HIP kernels with hipcc for gfx950.

Usage: python -m prefix_shared_kv_radix_amd.build   (or __graft_entry__.build()).
Always recompiles (a few seconds per kernel file, in parallel).
"""
from __future__ import annotations

import glob
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "radix_attn")
LIB = os.path.join(PKG, "libradix_attn.so")
ARCH = os.environ.get("RADIX_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no kernel produces or tests NaNs (masked scores are -inf): lets fmaxf map to
    # v_max3 without canonicalising each operand first
    "-fno-honor-nans",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


# Kernels whose private-tail ring counts its own loads for explicit s_waitcnt: any
# scratch access (a spill) inside them would shift those counts, so they must not spill.
NO_SCRATCH = re.compile(r"(tail_bf16_kernel|decode_fused_kernel)ILi[124]E")


def _check_scratch(report: str, src: str) -> None:
    """Reject a build in which a kernel matching NO_SCRATCH uses scratch memory."""
    name = None
    for line in report.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and NO_SCRATCH.search(name) and int(m.group(1)) > 0:
            raise RuntimeError(f"{src}: {name} spills ({m.group(1)} bytes/lane of scratch); "
                               "its explicit load waits would be wrong")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "host", "*.cpp"))):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", src, "-o", obj])
    for src in sorted(glob.glob(os.path.join(CSRC, "kernels", "*.hip"))):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src,
                     "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    for cmd, out in zip(jobs, outs):
        if cmd[0] == HIPCC:
            _check_scratch(out, cmd[-3])
    if verbose:
        for o in outs:
            for line in o.splitlines():
                if "remark" not in line:
                    print(line)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
