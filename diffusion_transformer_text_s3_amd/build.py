"""Build the gfx950 library libzdit.so in-tree: each HIP source under csrc/ is compiled with
hipcc for --offload-arch=gfx950 into _build/, then linked into lib/libzdit.so.

    python -m diffusion_transformer_text_s3_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libzdit.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, extra: list[str]) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name and says so; harmless
    log = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{log}")
    return obj, log


def build(verbose: bool = False, extra_flags: list[str] | None = None, jobs: int = 8) -> str:
    """Compile every source and link lib/libzdit.so; returns the library path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    extra = list(extra_flags or [])
    srcs = _sources()
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), srcs))
    objs = [o for o, _ in results]
    if verbose:
        for o, log in results:
            if log.strip():
                print(f"[{os.path.basename(o)}]\n{log}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    shutil.move(tmp, LIB)
    return LIB


SAN_FLAGS = ["-O1", "-g",
             # host code only: the device code is built as usual
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_DIR = os.path.join(BUILD, "asan")
SAN_LIB = os.path.join(SAN_DIR, "libzdit_asan.so")


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime (with the UndefinedBehaviorSanitizer handlers) that a
    process loading the sanitized library must preload."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        lib = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang")
        for v in sorted(os.listdir(lib)) if os.path.isdir(lib) else []:
            cand = os.path.join(lib, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
            if os.path.exists(cand):
                return cand
        raise RuntimeError("clang ASan runtime not found")
    return path


def build_sanitized(jobs: int = 8) -> str:
    """The host code of the library built with AddressSanitizer and UndefinedBehaviorSanitizer
    (device code unchanged) into _build/asan/libzdit_asan.so, for the host-side tests; not the
    product library."""
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = _sources()

    def one(src):
        obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
        cmd = [HIPCC, *[f for f in COMMON_FLAGS if f != "-O3"], *SAN_FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-o", SAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized())
    else:
        path = build(verbose="-v" in sys.argv)
        print(path)
