"""Build the HIP library libhybridattn.so in-tree for gfx950.

Every source is compiled with hipcc for gfx950 only, with packed-FP32
instruction generation disabled, into position-independent objects that are
linked into one shared library next to this file.

    python -m hybrid_sliding_window_gqa_amd.build
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_NAME = "libhybridattn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["api.cpp", "split_policy.cpp", "append.hip", "decode.hip", "prefill.hip", "verify.hip", "prefix_tree.cpp",
           "probe.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libhybridattn.so)")


def common_flags() -> list[str]:
    return [
        "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # keep MFMA accumulators in VGPRs: no AGPR copies around the softmax rescale
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
    ]


def build(verbose: bool = False) -> str:
    """Compile every source and link the library. Returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj])

    def run(cmd):
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        # hipcc's host pass does not know the packed-fp32 feature flag: harmless noise
        noise = "'-packed-fp32-ops' is not a recognized feature"
        err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return err

    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as pool:
        list(pool.map(run, cmds))
    tmp = LIB_PATH + ".tmp"
    run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    _check_kernel_stubs(tmp)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


HOST_SANITIZED_SOURCES = ["api.cpp", "split_policy.cpp", "prefix_tree.cpp", "sanitize_stubs.cpp"]
HOST_SANITIZED_DIR = os.path.join(BUILD_DIR, "host_sanitized")


def build_host_sanitized() -> str:
    """Host-only copy of the library for AddressSanitizer and
    UndefinedBehaviorSanitizer: the host sources built by the host compiler
    (no HIP code), the kernel launchers stubbed (sanitize_stubs.cpp). Returns
    the library path. The GPU library is not touched."""
    gxx = shutil.which("g++")
    if gxx is None:
        raise RuntimeError("g++ not found")
    os.makedirs(HOST_SANITIZED_DIR, exist_ok=True)
    out = os.path.join(HOST_SANITIZED_DIR, LIB_NAME)
    sanitize = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-Wall", "-Wno-unused-function",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), *sanitize,
           *[os.path.join(CSRC, s) for s in HOST_SANITIZED_SOURCES], "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"host sanitizer build failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return out


def _check_kernel_stubs(lib: str) -> None:
    """Fail when a kernel's host launch stub is referenced but not defined.

    clang's host pass can drop a kernel template instantiation without a
    diagnostic (for instance when a device-only construct inside it cannot be
    checked for the host); the library then links but cannot be loaded."""
    nm = shutil.which("nm")
    if nm is None:
        return
    res = subprocess.run([nm, "-D", "--undefined-only", lib], capture_output=True, text=True)
    missing = [line.split()[-1] for line in res.stdout.splitlines() if "__device_stub__" in line]
    if missing:
        raise RuntimeError("kernel launch stubs missing from the host objects: " + ", ".join(missing))


if __name__ == "__main__":
    print(build(verbose=True))
