"""Build libvit.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every HIP source under ``csrc/`` is compiled to an object in parallel, then
linked into ``vision_encoder_varlen_amd/libvit.so`` next to this file, where the
Python binding loads it.  The MFMA-rate probe under ``probe/`` (measurement
support, not part of the attention path) becomes a library of its own,
``libvit_probe.so``.  Packed-fp32 VALU instructions are disabled for the
device code.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libvit.so")
PROBE_SRC = os.path.join(HERE, "probe", "probe.hip")
PROBE_PATH = os.path.join(HERE, "libvit_probe.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libvit.so)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


# Host code instrumented with AddressSanitizer and UndefinedBehaviorSanitizer;
# the device code is built as usual.  -Xarch_host keeps each sanitizer off the
# GPU compilation.
HOST_SANITIZER_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
]


def clangxx() -> str:
    for cand in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("clang++ not found (needed to link the sanitizer build)")


def sanitizer_runtime() -> str:
    """Path of the shared AddressSanitizer runtime the sanitizer build links
    against (it also carries UndefinedBehaviorSanitizer); a process that loads
    that build must preload it."""
    res = subprocess.run([clangxx(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True)
    return res.stdout.strip()


def build_host_sanitized(out_path: str, verbose: bool = False) -> str:
    """Build a copy of the library whose host code (argument checks, scratch
    management, launches) runs under ASan + UBSan, for the CPU tests of the C
    ABI.  Objects go to their own folder; the link is a plain clang++ host
    link against the HIP runtime (every object already holds its device code)."""
    obj_dir = os.path.join(BUILD_DIR, "host_sanitized")
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        cmd = [hipcc(), *COMMON_FLAGS, *HOST_SANITIZER_FLAGS, "-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(hipcc())), "lib")
    cmd = [clangxx(), "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan",
           "-o", out_path, *objs, f"-L{rocm_lib}", "-lamdhip64", f"-Wl,-rpath,{rocm_lib}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(f"built {out_path}", file=sys.stderr)
    return out_path


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile and link libvit.so; returns its path.  Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    build_probe()
    if verbose:
        print(f"built {LIB_PATH} and {PROBE_PATH}", file=sys.stderr)
    return LIB_PATH


def build_probe() -> str:
    """Compile and link libvit_probe.so (the MFMA-rate probe); returns its path."""
    tmp = PROBE_PATH + ".tmp"
    cmd = [hipcc(), *COMMON_FLAGS, "-shared", "-o", tmp, PROBE_SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"probe build failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, PROBE_PATH)
    return PROBE_PATH


if __name__ == "__main__":
    build(verbose=True)
