"""Build libaqkv.so in-tree for gfx950 with hipcc.

    python -m kv_cache_compression_quantize_amd.build        # or build() from Python

Every call recompiles every source (a clean, complete build), objects go to
``_build/`` next to this file, the shared library to ``libaqkv.so`` beside it.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libaqkv.so")
ARCH = os.environ.get("AQKV_ARCH", "gfx950")

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]
# Device pass only.  A .hip source compiles in two steps: the device code to an offload
# bundle with these flags, then the host side with that bundle embedded; the target
# feature below is a gfx950 one that the host compiler would only warn about.
DEVICE_FLAGS = [
    # IEEE single-precision divide (value codes are decided by (v - min) / scale)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # never emit packed fp32 ALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix instructions read and write their accumulators in VGPRs (no AGPR copies
    # around the VALU work that shares them)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]

# per-file additions
FILE_FLAGS = {
    # min / max of finite inputs: no NaN quieting before each v_min / v_max, so
    # the DPP lane swaps fold into them
    "quant_values.hip": ["-fno-honor-nans"],
}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + p.stdout)
    return p.stdout


def _run_all(cmds):
    return "".join(_run(c) for c in cmds)


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        dev = os.path.join(BUILD, os.path.basename(src) + ".dev")
        flags = [*HIP_FLAGS, *FILE_FLAGS.get(os.path.basename(src), [])]
        jobs.append([
            [hipcc, *flags, *DEVICE_FLAGS, "--cuda-device-only", "-c", src, "-o", dev],
            [hipcc, *flags, "--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary", "-Xclang", dev,
             "-c", src, "-o", obj],
        ])
        objs.append(obj)
    for src in sorted(glob.glob(os.path.join(CSRC, "*.cpp"))):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        jobs.append([["g++", "-O2", "-fPIC", "-std=c++17", "-Wall", "-c", src, "-o", obj]])
        objs.append(obj)
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        outs = list(ex.map(_run_all, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
