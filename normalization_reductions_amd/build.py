"""Build libnormred.so (gfx950) in-tree with hipcc.

Every .hip/.cpp file under csrc/ is compiled to an object in parallel, then linked into
``normalization_reductions_amd/libnormred.so``. Device code targets gfx950 only and is built
with packed-FP32 instructions disabled (``-packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnormred.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def common_flags(debug: bool = False) -> list[str]:
    return [
        "-std=c++17", "-fPIC", "-O0" if debug else "-O3", "-g0",
        f"--offload-arch={ARCH}",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
        "-fvisibility=hidden",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _compile(src: str, debug: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags(debug) + ["-c", src, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    return obj


def build(debug: bool = False, jobs: int | None = None) -> str:
    """Compile all sources and link libnormred.so; returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, debug), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    return LIB


def build_host_asan(outdir: str) -> tuple[str, str]:
    """Debug builds of the host code for the sanitizer test: abi.cpp (the C ABI's validation,
    planning and dispatch) with g++ -O0 -g and AddressSanitizer + UndefinedBehaviorSanitizer,
    linked with the device objects of the last build() into libnormred_asan.so, and oracle.c
    the same way into liboracle_asan.so. Device code is not sanitized. Returns both paths."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    os.makedirs(outdir, exist_ok=True)
    san = ["-O0", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined"]
    abi_o = os.path.join(outdir, "abi_asan.o")
    lib = os.path.join(outdir, "libnormred_asan.so")
    orc = os.path.join(outdir, "liboracle_asan.so")
    dev_objs = sorted(glob.glob(os.path.join(OBJDIR, "*.hip.o")))
    if not dev_objs:
        raise RuntimeError("no device objects in %s: run build() first" % OBJDIR)
    steps = [
        ["g++", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
         "-I", INCLUDE, "-I", CSRC] + san + ["-c", os.path.join(CSRC, "abi.cpp"), "-o", abi_o],
        ["g++", "-shared", "-fsanitize=address,undefined", "-o", lib, abi_o] + dev_objs +
        ["-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")],
        ["gcc", "-std=c11", "-fPIC", "-shared", "-pthread"] + san +
        ["-o", orc, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"],
    ]
    for cmd in steps:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("sanitizer build failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    return lib, orc


if __name__ == "__main__":
    print(build())
