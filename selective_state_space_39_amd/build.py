"""Build libssm_scan.so for gfx950 with hipcc (in-tree, next to this file).

    python -m selective_state_space_39_amd.build [--asm DIR]

Every call compiles from source. ``--asm DIR`` also writes the gfx950
assembly of the kernels to DIR for inspection.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libssm_scan.so")
SOURCES = [os.path.join(CSRC, "s6_kernels.hip"), os.path.join(CSRC, "s6_bwd.hip"), os.path.join(CSRC, "ssd_kernels.hip"),
           os.path.join(CSRC, "ssm_api.cpp")]
ARCH = "gfx950"

# Packed FP32 (v_pk_fma_f32 and friends) stays off in every HIP file.
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(asm_dir: str | None = None, quiet: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-shared", "-x", "hip", *SOURCES, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    if not quiet:
        noise = "is not a recognized feature for this target"
        msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l and "ignoring feature" not in l)
        if msg.strip():
            print(msg, file=sys.stderr)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        for src in SOURCES[:3]:
            out = os.path.join(asm_dir, os.path.basename(src).replace(".hip", ".s"))
            subprocess.run([hipcc(), *FLAGS, "--cuda-device-only", "-S", "-x", "hip", src, "-o", out],
                           check=True, capture_output=True)
    return LIB


DEMO_SRC = os.path.join(ROOT, "tests", "c_abi", "scan_demo.cpp")
DEMO = os.path.join(ROOT, "tests", "c_abi", "scan_demo")


def build_demo() -> str:
    """The C-ABI example consumer the tests run (plain C++ and the HIP runtime,
    no Python): linked against the in-tree library, found through an rpath
    relative to the binary, so the tree can move."""
    rpath = "$ORIGIN/" + os.path.relpath(HERE, os.path.dirname(DEMO))
    cmd = [hipcc(), "-O2", "-std=c++17", "-Wall", f"--offload-arch={ARCH}", "-I", INCLUDE, DEMO_SRC, "-o", DEMO + ".tmp",
           "-L", HERE, "-lssm_scan", f"-Wl,-rpath,{rpath}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    os.replace(DEMO + ".tmp", DEMO)
    return DEMO


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None)
    args = ap.parse_args()
    print(build(args.asm))
    print(build_demo())
