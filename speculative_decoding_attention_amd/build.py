"""Builds libspecattn.so in-tree for gfx950 with hipcc.

    python -m speculative_decoding_attention_amd.build [--host-sanitizers]

Each HIP source is compiled in parallel to an object under ``_build/`` and
the objects are linked into ``speculative_decoding_attention_amd/libspecattn.so``.

``--host-sanitizers`` builds ``libspecattn_hostsan.so`` instead: the same
sources with AddressSanitizer and UndefinedBehaviorSanitizer on the host
code only (argument checks, planning, launch set-up; the gfx950 code is
built as usual).  The sanitizer runtime is linked as a shared library, so a
process that loads it must preload that runtime (``asan_runtime()``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libspecattn.so")
LIB_HOSTSAN = os.path.join(PKG, "libspecattn_hostsan.so")
SOURCES = ["api.hip", "attention.hip", "topk.hip", "hsr.hip", "accept.hip", "validate.hip", "std.hip",
           "stream.hip"]
ARCH = os.environ.get("SPEC_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from forming packed fp32 arithmetic on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
]
# host-only instrumentation: each -fsanitize= applies to the host pass alone
HOSTSAN = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libspecattn")


def asan_runtime() -> str:
    """Path of the shared AddressSanitizer runtime that hipcc links against."""
    res = subprocess.run([_hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime of hipcc's clang was not found")
    return path


def _compile(src: str, hipcc: str, build_dir: str, extra: list) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build_library(verbose: bool = False, host_sanitizers: bool = False) -> str:
    """Compile every HIP source and link libspecattn.so (or, with
    host_sanitizers, libspecattn_hostsan.so); returns its path."""
    hipcc = _hipcc()
    build_dir = os.path.join(BUILD, "hostsan") if host_sanitizers else BUILD
    extra = HOSTSAN if host_sanitizers else []
    lib = LIB_HOSTSAN if host_sanitizers else LIB
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, build_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    link_extra = ["-shared-libsan", *HOSTSAN] if host_sanitizers else []
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build_library(verbose=True, host_sanitizers="--host-sanitizers" in sys.argv[1:])
    sys.exit(0)
