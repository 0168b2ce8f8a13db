"""Build libengram.so in-tree with hipcc for gfx950.

    python gram_hash_memory_amd/build.py

(not `python -m`: importing the package loads the library this builds)

Each HIP source is compiled to an object file under _build/, in parallel, and
the objects are linked into gram_hash_memory_amd/libengram.so.  No GPU is
needed: hipcc cross-compiles the device code for gfx950.
"""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libengram.so")
SOURCES = ["api.cpp", "hash.hip", "rows.hip", "gemm.hip", "gemm_skinny.hip", "gemm_q2k.hip",
           "gemm_fp8.hip", "gemm_mx.hip", "mx_quant.hip", "gate.hip"]

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-mcode-object-version=5",
    # No packed-fp32 instructions: hipcc would otherwise form them from scalar code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-DENGRAM_BUILDING_LIBRARY",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def source_files() -> list[str]:
    """Every file the library is built from: kernels, headers and this script."""
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))
             if f.endswith((".hip", ".hpp", ".cpp", ".h"))]
    inc = os.path.join(ROOT, "include")
    files += [os.path.join(inc, f) for f in sorted(os.listdir(inc)) if f.endswith(".h")]
    return files + [os.path.abspath(__file__)]


def source_hash() -> str:
    """sha256 over the names and contents of source_files(), as hex."""
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.relpath(path, ROOT).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()


def build_id() -> str:
    """What engram_build_id() of a library built from the current sources returns."""
    return "sha256:" + source_hash()


def library_is_current() -> bool:
    """True if LIB exists and was built from the current sources (read from the
    file, without loading it)."""
    if not os.path.exists(LIB):
        return False
    with open(LIB, "rb") as f:
        return (b"engram-build-id " + build_id().encode() + b"\0") in f.read()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libengram.so)")


def _compile(src: str, bid: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    extra = [f'-DENGRAM_BUILD_ID="{bid}"'] if src == "api.cpp" else []
    cmd = [hipcc(), "-x", "hip", *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    return obj


# Host-side sanitizers for the ABI tests (the device code is built as usual;
# GPU sanitizers are not used).  Each flag applies to the host compilation only.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
SANITIZED_LIB = os.path.join(BUILD, "sanitized", "libengram_sanitized.so")


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime to preload into a host process."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin",
                         "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or "clang"
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    return res.stdout.strip()


def build_sanitized(verbose: bool = False) -> str:
    """libengram with AddressSanitizer and UndefinedBehaviorSanitizer in its host
    code, for running the host-side validation tests under the sanitizers."""
    out = os.path.dirname(SANITIZED_LIB)
    os.makedirs(out, exist_ok=True)
    bid = build_id()

    def comp(src):
        obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
        extra = [f'-DENGRAM_BUILD_ID="{bid}"'] if src == "api.cpp" else []
        cmd = [hipcc(), "-x", "hip", *FLAGS, *SANITIZE, *extra, "-c", os.path.join(CSRC, src),
               "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}{res.stderr}")
        return obj
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(comp, SOURCES))
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *SANITIZE, "-shared-libsan",
           *objs, "-o", SANITIZED_LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    if verbose:
        print("built", SANITIZED_LIB)
    return SANITIZED_LIB


def build(verbose: bool = False) -> str:
    """Compile every source and link libengram.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    for stale in os.listdir(BUILD):          # objects of sources that no longer exist
        if stale.endswith(".o") and stale[:-2] not in {os.path.splitext(f)[0] for f in SOURCES}:
            os.remove(os.path.join(BUILD, stale))
    bid = build_id()
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda src: _compile(src, bid), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)       # atomic: a process that already loaded the old file keeps it
    if verbose:
        print("built", LIB, bid)
    return LIB


if __name__ == "__main__":
    if "--sanitized" in sys.argv[1:]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
