"""Build the HIP library in-tree: weight_shared_rank_amd/libweightless.so.

Compiles every source under csrc/ for gfx950 with hipcc and links one shared
library exporting the C ABI declared in include/weightless.h.  Packed fp32
instructions are disabled for all device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libweightless.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["weightless.cpp", "decode.hip", "prefill.hip", "pack.hip", "decompose_kernels.hip", "decompose.cpp"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-x", "hip",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function",
         f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    if verbose and (r.stdout or r.stderr):
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        if out.strip():
            print(out)


def build(verbose=True, extra_flags=()):
    """Compile all sources and link libweightless.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        _run([HIPCC, *FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def asan_runtime():
    """Path of the clang AddressSanitizer runtime that a host-sanitized
    library needs preloaded into the (uninstrumented) Python process."""
    import glob
    found = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang", "*",
                                          "lib", "linux", "libclang_rt.asan-x86_64.so")))
    return found[-1] if found else None


def build_host_sanitized(verbose=False):
    """A copy of the library whose host code (the C ABI, the planners, the
    launchers, the decomposition driver) is built with AddressSanitizer and
    UndefinedBehaviorSanitizer; device code is built as usual (no GPU
    sanitizer).  Written to _build/asan/libweightless_asan.so; load it with
    asan_runtime() preloaded.  For CPU tests of the host paths only."""
    from concurrent.futures import ThreadPoolExecutor
    out = os.path.join(BUILD, "asan")
    os.makedirs(out, exist_ok=True)
    # host-side only: every sanitizer flag is preceded by -Xarch_host
    san = [flag for kind in ("address", "undefined") for flag in ("-Xarch_host", "-fsanitize=" + kind)]
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g", *san, "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = [os.path.join(out, os.path.splitext(src)[0] + ".o") for src in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda so: _run([HIPCC, *flags, "-c", os.path.join(CSRC, so[0]), "-o", so[1]], verbose),
                    zip(SOURCES, objs)))
    lib = os.path.join(out, "libweightless_asan.so")
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *san, "-shared-libsan", *objs, "-o", lib], verbose)
    return lib


if __name__ == "__main__":
    build(verbose=True)
