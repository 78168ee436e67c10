"""Build step of the vlbridge library: compiles the HIP sources for gfx950 into
patch_merge_mlp_amd/libvlbridge.so (in-tree, next to the binding)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libvlbridge.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-function",
        # no packed-fp32 instructions (v_pk_*_f32) in any kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def _compile(src: str, build_dir: str, verbose: bool) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *compile_flags(), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Always recompiles (this is the does-it-build check) and returns the .so path.
    The sources compile in parallel, at most 8 at a time."""
    from concurrent.futures import ThreadPoolExecutor
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, verbose), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-shared-libsan",
            "-Xarch_host", "-fno-omit-frame-pointer"]
HOST_SOURCES = ("vlb_api.hip", "vlb_processor.hip")  # argument checks, planner, launches


def build_sanitized(out_dir: str) -> str:
    """A build whose host code in HOST_SOURCES carries AddressSanitizer and
    UndefinedBehaviorSanitizer (the device code is unchanged; the other sources
    compile as usual).  Load it with the clang sanitizer runtime preloaded
    (sanitizer_runtime()); used by the CPU tests only."""
    from concurrent.futures import ThreadPoolExecutor

    def one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        extra = SANITIZE + ["-g"] if os.path.basename(src) in HOST_SOURCES else []
        cmd = [HIPCC, *compile_flags(), *extra, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-3000:]}")
        return obj

    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    so = os.path.join(out_dir, "libvlbridge_san.so")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-fsanitize=address,undefined",
           "-shared-libsan", "-o", so, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    return so


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime (it carries the UndefinedBehaviorSanitizer
    handlers too) that the sanitized builds need preloaded."""
    found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return found[-1]


if __name__ == "__main__":
    print(build(verbose=True))
