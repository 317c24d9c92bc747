"""Build step: compile the HIP sources for gfx950 into lib/libattn_gqa.so with hipcc.

Usage: python -m attention_gqa_flash_02_amd.build [--jobs N] [--verbose] [--asan]
Every call rebuilds (objects go to lib/_build/, one hipcc process per source, then one link).
--asan also builds lib/libattn_gqa_asan.so: the same sources with AddressSanitizer on the host
code only (the GPU code is built as usual, at -O1), for the host-side validation tests; it is
loaded through ATTN_GQA_LIBRARY with the clang ASan runtime preloaded.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
BUILD = os.path.join(LIBDIR, "_build")
LIB = os.path.join(LIBDIR, "libattn_gqa.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # never emit packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
]


LIB_ASAN = os.path.join(LIBDIR, "libattn_gqa_asan.so")
BUILD_ASAN = os.path.join(LIBDIR, "_build_asan")
# host code only: each sanitizer flag is preceded by -Xarch_host
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, verbose, asan=False):
    obj = os.path.join(BUILD_ASAN if asan else BUILD, os.path.basename(src) + ".o")
    flags = [f for f in CXXFLAGS if f != "-O3"] + ["-O1", "-g"] + ASAN_FLAGS if asan else CXXFLAGS
    cmd = [HIPCC, *flags, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(x for x in (r.stdout + r.stderr).splitlines()
                    if "unknown target feature" not in x and "packed-fp32-ops" not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    return obj, msg


def build(jobs=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), srcs))
    objs = [o for o, _ in results]
    for _, msg in results:
        if verbose and msg.strip():
            print(msg)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def build_asan(jobs=None, verbose=False):
    """lib/libattn_gqa_asan.so: host code under AddressSanitizer (see the module docstring)."""
    os.makedirs(BUILD_ASAN, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose, asan=True), srcs))
    tmp = LIB_ASAN + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *ASAN_FLAGS[:2], "-shared-libsan", "-o", tmp,
           *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_ASAN)
    return LIB_ASAN


def asan_runtime():
    """Path of the clang AddressSanitizer runtime that LIB_ASAN links against, or None."""
    r = subprocess.run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip().splitlines()[-1] if r.returncode == 0 and r.stdout.strip() else ""
    return path if os.path.isabs(path) and os.path.exists(path) else None


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--asan", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
    if a.asan:
        print(build_asan(a.jobs, a.verbose))
    sys.exit(0)
