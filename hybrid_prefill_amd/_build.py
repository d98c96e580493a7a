"""Compile libhypic.so for gfx950 with hipcc (in-tree, next to this file)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libhypic.so")
OBJ_DIR = os.path.join(HERE, "_build")

SOURCES = ["hypic_abi.hip", "build_ref.hip", "build_mfma.hip", "build_fwd_mfma.hip", "build_sd_mfma.hip",
           "compose_ref.hip",
           "compose_mfma.hip", "conv_warmup.hip", "conv_kv.hip",
           "build_kda.hip", "build_kda_mfma.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 math (v_pk_*_f32): keep every fp32 op scalar
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


# measured-peak microbenchmarks for the benchmark (a library of their own, outside the ABI)
PEAKS_SOURCES = ["peaks.hip"]
PEAKS_LIB = os.path.join(HERE, "libhypic_peaks.so")


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


# Host-sanitized copy of the library for the CPU sanitizer test: the ABI translation
# unit (argument validation, dispatch) is compiled with AddressSanitizer and
# UndefinedBehaviorSanitizer on its host side only, and linked with the kernels'
# ordinary objects.  A process loads it with clang's ASan runtime preloaded.
SAN_LIB = os.path.join(HERE, "libhypic_san.so")
SAN_FLAGS = ["-g", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]


def build_sanitized(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    san_obj = os.path.join(OBJ_DIR, "hypic_abi_san.o")
    cmd = [HIPCC, *FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, "hypic_abi.hip"), "-o", san_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on hypic_abi.hip (sanitized)")
    objs = [san_obj] + [os.path.join(OBJ_DIR, s.replace(".hip", ".o")) for s in SOURCES if s != "hypic_abi.hip"]
    for o in objs[1:]:
        if not os.path.exists(o):
            raise RuntimeError(f"{o} is missing: run build() first")
    tmp = SAN_LIB + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    *objs, "-o", tmp], check=True)
    os.replace(tmp, SAN_LIB)
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(PEAKS_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + PEAKS_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PEAKS_LIB)
    if verbose:
        print("built", LIB, "and", PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
