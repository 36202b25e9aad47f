"""Build libkaio.so (the gfx950 HIP kernels plus the C ABI) in-tree with hipcc.

    python -m int4_group_quantized_w4a16_amd.build_lib
    python -m int4_group_quantized_w4a16_amd.build_lib --host-sanitizers

The second form builds _build/sanitize/libkaio.so: the same kernels, with the
host-side ABI layer (validation, device check, dispatch) instrumented by
AddressSanitizer and UndefinedBehaviorSanitizer (host code only; the GPU code
is built as usual).  Run the CPU boundary tests against it with

    LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1 \
    KAIO_LIBRARY=$PWD/int4_group_quantized_w4a16_amd/_build/sanitize/libkaio.so \
    python -m pytest tests/test_abi_host.py
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkaio.so")
SOURCES = ["kaio_abi.cpp", "qkv_prefill.hip", "qkv_decode.hip", "gemm_f16f32.hip", "dequant_group_bwd.hip"]
# measurement aid for the benchmark (a plain streaming read), a library of its own
ROOF_LIB = os.path.join(PKG, "libkaio_roof.so")
ROOF_SOURCES = ["roof.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep packed-FP32 VALU ops out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


# host-only sanitizer flags: each one behind -Xarch_host so that no GPU code is instrumented
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-g"]


def build_host_sanitized(verbose: bool = False) -> str:
    """libkaio.so with the host ABI layer under ASan/UBSan, in _build/sanitize/ (CPU testing only)."""
    out = os.path.join(BUILD, "sanitize")
    os.makedirs(out, exist_ok=True)
    objs = []
    for src in SOURCES:
        stem = os.path.splitext(src)[0] + ".o"
        plain = os.path.join(BUILD, stem)
        if not src.endswith(".cpp") and os.path.exists(plain) and \
                os.path.getmtime(plain) >= os.path.getmtime(os.path.join(CSRC, src)):
            objs.append(plain)        # GPU sources: the regular build's object, unchanged
            continue
        obj = os.path.join(out, stem)
        extra = HOST_SANITIZE if src.endswith(".cpp") else []
        cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    lib = os.path.join(out, "libkaio.so")
    _link(objs, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build(extra_flags=(), verbose: bool = False) -> str:
    """Compile every source for gfx950, link libkaio.so (and the benchmark's
    libkaio_roof.so); returns the path of libkaio.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + ROOF_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], ROOF_LIB)
    if verbose:
        print(f"built {LIB} and {ROOF_LIB}")
    return LIB


if __name__ == "__main__":
    if sys.argv[1:] == ["--host-sanitizers"]:
        build_host_sanitized(verbose=True)
    else:
        build(extra_flags=sys.argv[1:], verbose=True)
