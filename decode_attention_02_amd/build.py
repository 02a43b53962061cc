"""Build libmfa.so (and the benchmark's stream probe, libmfa_probe.so)
in-tree with hipcc for gfx950.

Usage: ``python -m decode_attention_02_amd.build`` (or ``build()``). Every
call compiles from source; the result lands next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmfa.so")
# measurement aid for bench.py (a pure read stream), built beside the library
PROBE = os.path.join(HERE, "libmfa_probe.so")
PROBE_SOURCES = ["stream_probe.hip"]

SOURCES = ["mfa_api.cpp", "attn_mfma.hip", "attn_valu.hip", "combine.hip", "kv_append.hip",
           "qproj.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: cannot build libmfa.so")
    return exe


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC, "-x", "hip", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    psrcs = [os.path.join(CSRC, s) for s in PROBE_SOURCES]
    cmd = [hipcc(), *FLAGS, "-x", "hip", *psrcs, "-o", PROBE + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(PROBE + ".tmp", PROBE)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
