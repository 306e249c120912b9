"""Build libpkv.so in-tree with hipcc for gfx950.

    python paged_kv_cache_459_amd/build.py          # compile (always) and link

Run it as a file (not ``-m``): importing the package would load the library it rebuilds.

Objects go to ``_build/`` at the repository root; the library to
``paged_kv_cache_459_amd/libpkv.so``. All HIP code is compiled with packed-FP32 instructions
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkv.so")
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")

HIP_SOURCES = ["pkv_attn.hip", "pkv_write.hip", "pkv_prefill.hip", "pkv_probe.hip"]
HOST_SOURCES = ["pkv_api.cpp", "pkv_alloc.cpp", "pkv_plan.cpp", "pkv_engine.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result", "-Werror=inline-asm",
          f"-I{INCLUDE}"]
# Code-object v5: the library runs inside PyTorch's bundled HIP runtime, which can be older than
# this compiler (ROCm 7.0 beside a ROCm 7.2 toolchain); v5 is the version that runtime
# generation itself emits and loads.
DEVICE = [f"--offload-arch={ARCH}", "-mcode-object-version=5",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: install ROCm or put hipcc on PATH")
    return path


def _compile(src, is_hip):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c", src, "-o", obj] + COMMON
    if is_hip:
        cmd = [hipcc(), "-x", "hip", "-c", src, "-o", obj] + COMMON + DEVICE
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj, res.stderr


def build(verbose=False):
    """Compile every source and link libpkv.so. Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(os.path.join(CSRC, s), True) for s in HIP_SOURCES]
    jobs += [(os.path.join(CSRC, s), False) for s in HOST_SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda j: _compile(*j), jobs))
    objs = [r[0] for r in results]
    if verbose:
        for _, err in results:
            noise = "is not a recognized feature for this target"
            lines = [ln for ln in err.splitlines() if noise not in ln]
            if lines:
                print("\n".join(lines), file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-o", tmp] + objs + [f"--offload-arch={ARCH}", "-fPIC",
                                                    "-mcode-object-version=5"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


def ensure_built():
    """Build only if the library is missing (tests and tools call this)."""
    if not os.path.exists(LIB):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
