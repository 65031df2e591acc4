"""Build libgq.so (the C-ABI HIP library) for gfx950 in-tree.

    python -m post_weight_quantization_gq_amd.build [--asan]

compiles every csrc/*.hip into an object with hipcc and links
post_weight_quantization_gq_amd/_lib/libgq.so.  Every call recompiles.

With --asan it also links _lib/libgq_asan.so, the same library with AddressSanitizer
on the host code only (the device code is built as usual).  It leaves the sanitizer's
symbols to the runtime, so a process loads it with that runtime preloaded
(LD_PRELOAD=asan_runtime()) and selects it with GQ_LIBRARY=<path>; the argument
checks, workspace sizing and error reporting of the C ABI then run under the
sanitizer on the CPU.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libgq.so")
LIB_ASAN = os.path.join(LIBDIR, "libgq_asan.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]
# host-side AddressSanitizer (GPU sanitizers are not used)
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host compiler pass does not know the device-only target feature
    out = "\n".join(l for l in proc.stdout.splitlines()
                    if "packed-fp32-ops" not in l or "error" in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def asan_runtime() -> str | None:
    """The AddressSanitizer runtime of the ROCm compiler, or None."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build(verbose: bool = False, asan: bool = False) -> str:
    """Compile and link libgq.so (and, with asan, libgq_asan.so); returns libgq.so's path."""
    hipcc = _hipcc()
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    variants = [("_build", [], LIB)]
    if asan:
        variants.append(("_build_asan", ASAN_FLAGS, LIB_ASAN))
    jobs = []
    for objdir, extra, _ in variants:
        os.makedirs(os.path.join(PKG, objdir), exist_ok=True)
        for src in srcs:
            obj = os.path.join(PKG, objdir, os.path.basename(src)[:-4] + ".o")
            jobs.append([hipcc, *HIPCC_FLAGS, *extra, "-c", "-o", obj, src])

    with ThreadPoolExecutor(max(1, min(len(jobs), os.cpu_count() or 1))) as ex:
        outs = list(ex.map(_run, jobs))
    for objdir, _, lib in variants:
        objs = [os.path.join(PKG, objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
        tmp = lib + ".tmp"
        outs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]))
        os.replace(tmp, lib)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv, asan="--asan" in sys.argv)
    print(path)
