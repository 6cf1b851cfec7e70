"""Builds libfocus.so (the HIP kernels + C ABI) for gfx950 in-tree with hipcc.

Every .hip/.cpp file under csrc/ is compiled to an object in _build/ (in parallel), then linked
into decodability_aware_token_amd/libfocus.so.  All device code is compiled with packed-f32
instructions disabled.

`build_sanitized()` builds the same sources with AddressSanitizer and UndefinedBehaviorSanitizer
on the host code only (the device code is unchanged) into _build/sanitized/libfocus.so, for the
CPU-only ABI tests: load it with the sanitizer runtime preloaded (`sanitizer_runtime()`) and
FOCUS_LIBRARY pointing at it.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfocus.so")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


# host-only sanitizers: each flag applies to the host compilation, never to gfx950 code
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libasan"]
SANITIZED_DIR = os.path.join(BUILD, "sanitized")


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime that a sanitized library needs preloaded."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True)
    return res.stdout.strip()


def build_sanitized(verbose: bool = False) -> str:
    """The library with sanitized host code, in _build/sanitized/ (not the product library)."""
    return build(verbose, out_dir=SANITIZED_DIR, extra=SANITIZE)


def build(verbose: bool = False, out_dir: str = BUILD, extra=()) -> str:
    os.makedirs(out_dir, exist_ok=True)
    hipcc = _hipcc()
    lib = LIB if out_dir == BUILD else os.path.join(out_dir, "libfocus.so")

    def compile_one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        cmd = [hipcc, *COMMON, *extra, "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                        if "packed-fp32-ops' is not a recognized feature" not in l)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, sources()))
    tmp = lib + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
