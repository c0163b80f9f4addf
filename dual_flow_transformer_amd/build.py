"""Compile the HIP sources into the in-tree C-ABI library (gfx950).

    python -m dual_flow_transformer_amd.build

Every HIP translation unit is compiled with packed-fp32 instructions turned
off (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libdualflow.so")
SYNTH_DEV = os.path.join(ROOT, "synth", "_gen_dev.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + out)
    return out


def build_library(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip"))) + [os.path.join(PKG, "csrc", "api.cpp")]
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        futs = [ex.submit(_run, [HIPCC, *FLAGS, "-c", s, "-o", o]) for s, o in zip(srcs, objs)]
        for f in futs:
            out = f.result()
            if verbose and out:
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def build_synth_device() -> str:
    src = os.path.join(ROOT, "synth", "gen_dev.hip")
    tmp = SYNTH_DEV + ".tmp"
    _run([HIPCC, *FLAGS, "-shared", "-o", tmp, src])
    os.replace(tmp, SYNTH_DEV)
    return SYNTH_DEV


def build_all(verbose: bool = False):
    sys.path.insert(0, ROOT)
    import synth
    synth.build_host(force=True)
    build_synth_device()
    return build_library(verbose)


if __name__ == "__main__":
    print(build_all(verbose=True))
