"""Build ``libts.so`` (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m long_context_kv_ts_amd.build        # or __graft_entry__.build()

Each source compiles to an object under ``long_context_kv_ts_amd/_build`` with
hipcc, then the objects link into ``long_context_kv_ts_amd/libts.so``.
Packed fp32 instructions are disabled for every device compile.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libts.so")
# measurement probes of the benchmark (matrix-core and vector-ALU rates, HBM
# streaming read), kept out of the hot-path library
PROBE_LIB = os.path.join(PKG, "libts_probe.so")
PROBE_SOURCES = ["probe.hip"]
ARCH = "gfx950"
SOURCES = ["api.cpp", "attn_valu.hip", "attn_mfma.hip", "attn_small.hip", "attn_merge.hip",
           "importance.hip", "topk.hip", "gather.hip", "accept.hip", "tree.hip", "sample.hip", "ngram.hip",
           "fused.hip", "noalloc.hip"]
# Per-source extra flags. The matrix-core verify kernel never produces or
# consumes NaN (masked scores are -inf, every exp2 argument is finite or -inf),
# so it is built without NaN semantics: maxima of matrix-core results then need
# no quieting instruction and fuse into v_max3_f32.
EXTRA_FLAGS = {"attn_mfma.hip": ["-fno-honor-nans"], "sample.hip": ["-fno-honor-nans"]}


def _hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def _compile(src: str, hipcc: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc, *_flags(), *EXTRA_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str, hipcc: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


# Host-sanitized variant of the library for the CPU tests of the C ABI: api.cpp
# (argument checks, work planning, workspace carving) built with AddressSanitizer
# and UndefinedBehaviorSanitizer on its host code only, linked with the same
# kernel objects. Loading it needs the sanitizer runtime preloaded
# (tests/test_abi_sanitized.py does that in a child process).
SAN_DIR = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(SAN_DIR, "libts_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitized(hipcc: str | None = None, verbose: bool = True) -> str:
    """Build SAN_LIB from api.cpp (sanitized) and the kernel objects of build()."""
    hipcc = hipcc or _hipcc()
    os.makedirs(SAN_DIR, exist_ok=True)
    obj = os.path.join(SAN_DIR, "api_san.o")
    cmd = [hipcc, "-O1", "-g", *[f for f in _flags() if f != "-O3"], *SAN_FLAGS, "-c",
           os.path.join(CSRC, "api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    objs = [obj] + [os.path.join(OUT_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "api.cpp"]
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS[:4], "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def build(verbose: bool = True) -> str:
    hipcc = _hipcc()
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, hipcc), srcs)))
    _link([objs[s] for s in SOURCES], LIB, hipcc)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB, hipcc)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    build_host_sanitized(hipcc, verbose)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
