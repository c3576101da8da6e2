"""Build libmoe.so in-tree for gfx950.

Every source under ``csrc/`` is compiled with ``hipcc --offload-arch=gfx950``
and the objects are linked against the HIP runtime that PyTorch ships
(``torch/lib/libamdhip64.so``), so that the library and PyTorch share one
HIP runtime, one device context and one set of streams in the process.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libmoe.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

COMMON_FLAGS = [
    "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
HIP_FLAGS = [
    "--offload-arch=gfx950",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
]


def _torch_lib_dir() -> str:
    import torch  # noqa: WPS433 (build-time only)
    return os.path.join(os.path.dirname(torch.__file__), "lib")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("command failed:\n  " + " ".join(cmd) + "\n" + p.stdout)
    return p.stdout


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer build of the
# library (libmoe_asan.so) for the CPU tests of its host code: every
# sanitizer flag applies to the host compilation only (-Xarch_host); device
# code is built as usual.
ASAN_LIB_PATH = os.path.join(HERE, "libmoe_asan.so")
ASAN_BUILD_DIR = os.path.join(ROOT, "_build_asan")
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The compiler's shared ASan runtime (to preload into the interpreter)."""
    return _run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"]).strip()


def build(verbose: bool = False, jobs: int = 8, sanitize: bool = False) -> str:
    """Compile every source and link libmoe.so (libmoe_asan.so with
    sanitize).  Returns the library path."""
    bdir = ASAN_BUILD_DIR if sanitize else BUILD_DIR
    lib_path = ASAN_LIB_PATH if sanitize else LIB_PATH
    extra = SANITIZE_HOST if sanitize else []
    os.makedirs(bdir, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        if src.endswith(".hip"):
            cmd = [HIPCC, "-c", "-x", "hip", src, "-o", obj] + COMMON_FLAGS + HIP_FLAGS + extra
        else:
            cmd = [HIPCC, "-c", src, "-o", obj] + COMMON_FLAGS + extra
        out = _run(cmd)
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, srcs))
    tlib = _torch_lib_dir()
    tmp = lib_path + ".tmp"
    link_san = ["-fsanitize=address,undefined", "-shared-libasan"] if sanitize else []
    cmd = [CLANGXX, "-shared", "-fPIC", "-o", tmp] + objs + link_san + [
        "-L", tlib, "-l:libamdhip64.so", "-l:libhsa-runtime64.so", "-Wl,-rpath," + tlib,
        "-lstdc++", "-lm", "-lpthread",
    ] + ([] if sanitize else ["-Wl,--no-undefined"])
    out = _run(cmd)
    if verbose and out.strip():
        print(out)
    shutil.move(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
