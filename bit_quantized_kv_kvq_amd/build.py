"""Build libkvq.so for gfx950 with hipcc (in-tree; the .so ships with the sources).

    python -m bit_quantized_kv_kvq_amd.build [--jobs N]
    python -m bit_quantized_kv_kvq_amd.build --sanitize

--sanitize builds _build/san/libkvq_san.so instead: the host code of the
sources with host code in them (the C ABI, launch planning, validation) under
AddressSanitizer and UndefinedBehaviorSanitizer (-Xarch_host: the gfx950 code is
built as usual), linked with the kernels of a normal build.  A process loads it
with the clang ASan runtime preloaded (sanitizer_runtime() names it), e.g.

    LD_PRELOAD=$(python -c "import bit_quantized_kv_kvq_amd.build as b; print(b.sanitizer_runtime())") \
    ASAN_OPTIONS=detect_leaks=0 KVQ_LIB=bit_quantized_kv_kvq_amd/_build/san/libkvq_san.so \
    python -m pytest tests/test_lib_host.py
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


# sources whose host code does more than register kernels
HOST_SOURCES = ["kvq_host.cpp", "quant.hip", "decode.hip", "probe.hip"]
SAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime to preload for libkvq_san.so."""
    out = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    if not os.path.isabs(out):
        raise RuntimeError("no clang ASan runtime found")
    return out


def build_sanitized(jobs: int | None = None) -> str:
    """_build/san/libkvq_san.so: HOST_SOURCES with host-side ASan + UBSan, the other
    objects from a normal build (built first if missing)."""
    san = os.path.join(BUILD, "san")
    os.makedirs(san, exist_ok=True)
    if not all(os.path.exists(os.path.join(BUILD, os.path.splitext(s)[0] + ".o")) for s in SOURCES):
        build(jobs, verbose=False)

    def one(src):
        obj = os.path.join(san, os.path.splitext(src)[0] + ".o")
        flags = [f for f in FLAGS if f != "-O3"]
        cmd = [HIPCC, *flags, *SAN_FLAGS, *(DECODE_FLAGS if src.startswith("decode") else []),
               *(["-x", "hip"] if src.endswith(".cpp") else []), "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, res.stderr))
        return obj

    with cf.ThreadPoolExecutor(jobs or len(HOST_SOURCES)) as ex:
        objs = list(ex.map(one, HOST_SOURCES))
    objs += [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s not in HOST_SOURCES]
    out = os.path.join(san, "libkvq_san.so")
    subprocess.check_call([HIPCC, "--offload-arch=" + ARCH, "-shared", "-shared-libsan", "-Xarch_host",
                           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", out, *objs])
    print("built", out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--sanitize", action="store_true")
    args = ap.parse_args()
    if args.sanitize:
        build_sanitized(args.jobs)
    else:
        build(args.jobs)
