"""Build libssm.so (HIP, gfx950) in-tree with hipcc.

Every source under ``csrc/`` is compiled to an object in parallel, then linked
into ``selective_state_space_70_amd/libssm.so``. Device code is compiled for
gfx950 only, with packed-fp32 instruction selection disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libssm.so")
SOURCES = ["capi.hip", "plan.cpp", "scan_fwd.hip", "scan_fwd_n16.hip", "scan_fwd_n32.hip", "scan_fwd_n64.hip", "scan_bwd.hip", "ssd_fwd.hip", "ssd_bwd.hip", "decode.hip", "conv1d.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I" + INCLUDE, "-I" + CSRC,
]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the device-only feature flag
        text = "\n".join(l for l in text.splitlines()
                         if "packed-fp32-ops' is not a recognized feature" not in l)
        if text.strip() and (verbose or p.returncode):
            print(text, file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: %s" % ", ".join(failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
