"""Build libkvq.so for gfx950 with hipcc (in-tree; the .so ships with the sources).

    python -m bit_quantized_kv_kvq_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# the decode instantiations first: they take longest
SOURCES = ["decode_mf_b4_d128.hip", "decode_mf_b2_d128.hip", "decode_mf_b4_d64.hip", "decode_mf_b2_d64.hip",
           "decode_mf_b8_d128.hip", "decode_mf_b8_d64.hip",
           "decode_b4_d128.hip", "decode_b2_d128.hip", "decode_b4_d64.hip", "decode_b2_d64.hip",
           "decode_sp_b4_d128.hip", "decode_sp_b2_d128.hip", "decode_sp_b4_d64.hip", "decode_sp_b2_d64.hip",
           "decode_mfsp_b4_d128.hip", "decode_mfsp_b2_d128.hip",
           "decode_kt_b4_d128.hip", "decode_kt_b2_d128.hip", "decode_kt_b8_d128.hip",
           "decode_kt_b4_d64.hip", "decode_kt_b2_d64.hip", "decode_kt_b8_d64.hip",
           "kvq_host.cpp", "quant.hip", "decode.hip", "probe.hip"]

# -packed-fp32-ops: no packed fp32 VALU instructions anywhere.
# correctly rounded fp32 division: the codec divides exactly as IEEE binary32.
# No fast-math and no denormal flushing.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
         "-ffp-contract=fast-honor-pragmas"]


# Decode kernels: no NaN semantics needed (max reductions then skip canonicalising
# their operands).  The quantizer keeps IEEE behaviour.
DECODE_FLAGS = ["-fno-honor-nans"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS]
    if src.startswith("decode_"):
        cmd += DECODE_FLAGS
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every source and link libkvq.so.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=" + ARCH, "-shared", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    build(ap.parse_args().jobs)
