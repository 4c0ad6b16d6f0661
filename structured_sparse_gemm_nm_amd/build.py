"""Build libnmsparse.so in-tree with hipcc for gfx950.

    python -m structured_sparse_gemm_nm_amd.build [--sanitize]

Compiles every source under csrc/ to an object in parallel, then links the
shared library next to this file.  Always rebuilds.

--sanitize also links _build/libnmsparse_san.so: the same device objects with
the host-side C ABI (nm_api.cpp) built under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; the GPU code is not
instrumented).  Load it with NMSPARSE_LIB pointing at it and the clang ASan
runtime (SANITIZER_RUNTIME) preloaded.
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
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libnmsparse.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

# Every HIP translation unit is built without packed fp32 instructions.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
                "-Wall", "-Wno-unused-function"]
# Translation units whose MFMA loops hold every accumulator in VGPRs: without
# this the register allocator moves some accumulators between AGPRs and VGPRs
# every K step, and each move waits for the MFMA that wrote the value.
PER_SOURCE_FLAGS = {
    "nm_spmm_lds.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (looked in $HIPCC, /opt/rocm/bin, PATH)")


def sources():
    out = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".cpp")):
            out.append(os.path.join(CSRC, name))
    return out


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    extra = PER_SOURCE_FLAGS.get(os.path.basename(src), [])
    cmd = [hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), *COMMON_FLAGS, "-x", "hip", *DEVICE_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    warnings = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if warnings:
        sys.stderr.write("\n".join(warnings) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")) or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources")
    return LIB_PATH


SAN_LIB_PATH = os.path.join(BUILD_DIR, "libnmsparse_san.so")
SANITIZER_RUNTIME = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"
# each sanitizer flag applies to the host compilation only
SAN_HOST_FLAGS = ["-O1", "-g",
                  "-Xarch_host", "-fsanitize=address",
                  "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized(verbose: bool = True) -> str:
    """Link SAN_LIB_PATH: nm_api.cpp host-sanitized, every other object as built."""
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    api = os.path.join(CSRC, "nm_api.cpp")
    san_obj = os.path.join(BUILD_DIR, "nm_api.cpp.san.o")
    flags = [f for f in COMMON_FLAGS if f != "-O3"]
    cmd = [hipcc(), *flags, *SAN_HOST_FLAGS, "-x", "hip", *DEVICE_FLAGS, "-c", api, "-o", san_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    link = [o for o in objs if not o.endswith("nm_api.cpp.o")] + [san_obj]
    # the sanitizer runtime is not linked in: it is preloaded into the process
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", SAN_LIB_PATH, *link]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(f"built {SAN_LIB_PATH} (host ASan + UBSan)")
    return SAN_LIB_PATH


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized()
    else:
        build()
