"""Build libcomba.so (HIP, gfx950) in-tree with hipcc.

Run as ``python -m bilinear_rnn_amd.build``. Each .hip source compiles to an
object in parallel, then the objects link into one shared library next to
this file. Packed-fp32 instructions are disabled for device code.
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
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcomba.so")
OBJDIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Extra flags for single sources. The matrix-core ceiling kernel keeps its
# accumulators in ordinary VGPRs: with accumulation registers the allocator
# shuffles them between the MFMAs of its loop, which lowers the ceiling it
# is there to measure.
FILE_FLAGS = {"measure.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libcomba.so")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src).replace(".hip", ".o"))
    cmd = [_hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-side address and undefined-behaviour sanitizers for the CPU checks of
# the C ABI (argument validation, workspace carving): each -fsanitize flag
# applies to the host pass only, device code is built as usual.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized(out_dir: str) -> str:
    """libcomba.so with the host code under ASan and UBSan, written to
    out_dir/libcomba_san.so. Load it through COMBA_LIBRARY with the compiler's
    ASan runtime preloaded (sanitizer_runtime())."""
    os.makedirs(out_dir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"] + SANITIZE_HOST

    def one(src):
        obj = os.path.join(out_dir, os.path.basename(src).replace(".hip", ".o"))
        res = subprocess.run([_hipcc(), *flags, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj],
                             stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources()))) as ex:
        objs = list(ex.map(one, sources()))
    lib = os.path.join(out_dir, "libcomba_san.so")
    subprocess.check_call([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", lib, *objs])
    return lib


def sanitizer_runtime() -> str:
    """The compiler's shared ASan runtime (it carries the UBSan handlers too)."""
    out = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                         stderr=subprocess.DEVNULL, text=True).stdout.strip()
    if not out or not os.path.isabs(out) or not os.path.exists(out):
        import glob
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        out = hits[0] if hits else ""
    return out


if __name__ == "__main__":
    build()
