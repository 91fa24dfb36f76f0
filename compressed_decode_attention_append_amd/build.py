"""Build libtq.so (HIP kernels for gfx950 + C ABI + host codebook builder).

Usage: python -m compressed_decode_attention_append_amd.build [--debug]

Compiles every source under csrc/ with hipcc for gfx950 into _build/ at the
repository root and links the shared library next to this file.  Packed
fp32 VALU instructions are disabled for all device code.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtq.so")

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libtq needs the ROCm toolchain")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


# Per-source flags.  The decode kernel never sees NaN scores (infinities,
# which mark masked positions, keep their meaning), so its max reductions
# need not quiet NaNs first.
EXTRA_FLAGS = {"decode_mfma.hip": ["-fno-honor-nans"]}


def compile_one(src: str, debug: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + (["-x", "hip"] if src.endswith(".hip") else []) + ["-c", src, "-o", obj, "-fPIC", "-std=c++17",
           "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]
    cmd += ["-O1", "-g"] if debug else ["-O3"]
    if src.endswith(".hip"):
        cmd += [f"--offload-arch={ARCH}",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    cmd += EXTRA_FLAGS.get(os.path.basename(src), [])
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(debug: bool = False, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: compile_one(s, debug), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--debug", action="store_true")
    a = ap.parse_args()
    build(debug=a.debug)
