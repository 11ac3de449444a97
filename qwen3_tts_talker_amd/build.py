"""Build ``libqtalk.so`` (the C-ABI library) in-tree with hipcc for gfx950.

Run ``python -m qwen3_tts_talker_amd.build``; every call recompiles.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqtalk.so")
SOURCES = ["runtime.cpp", "k_gemv.hip", "k_attn.hip", "k_gemm.hip", "k_attn_prefill.hip",
           "k_decode_fused.hip", "k_frame.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed float32 instructions stay off: hipcc would otherwise emit them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
]
# per-source extras: the persistent decode spends its time in short polling
# loops, whose speed measured sensitive to where they fall in the
# instruction stream; 64-byte loop alignment makes it independent of that
# the prefill attention produces no NaN (masked scores are -inf, every
# difference of infinities is guarded), so its maxima need no NaN-quieting
# canonicalisation of the score registers (about 15 fewer vector
# instructions per 32-key tile)
SOURCE_FLAGS = {"k_decode_fused.hip": ["-falign-loops=64"], "k_attn_prefill.hip": ["-fno-honor-nans"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build_library(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    with tempfile.TemporaryDirectory(prefix="qtalk_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        cmds = [[HIPCC, *FLAGS, *SOURCE_FLAGS.get(s, []), "-x", "hip", "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            for out in ex.map(_run, cmds):
                if verbose and out.strip():
                    print(out)
        tmp_lib = LIB + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib])
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
