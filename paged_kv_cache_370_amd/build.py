"""Build libpagedkv.so (HIP, gfx950) in-tree with hipcc.

    python -m paged_kv_cache_370_amd.build          # or build() from Python

Every translation unit is compiled in parallel to an object file under
_build/, then linked into paged_kv_cache_370_amd/libpagedkv.so.
"""

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep hipcc from forming packed fp32 arithmetic on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the online softmax rescales them with
    # vector ALU ops every chunk, and AGPRs would need copies both ways
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # single-lane atomics (work-queue claims) are not worth a wave-wide
    # expansion, whose result read-back forces a wait on all pending loads
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; install ROCm or put hipcc on PATH")
    return path


def _compile(src, obj):
    cmd = [_hipcc(), *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warnings = "\n".join(line for line in r.stderr.splitlines()
                         if "packed-fp32-ops" not in line and line.strip())
    return obj, warnings


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        for obj, warn in ex.map(lambda so: _compile(*so), zip(srcs, objs)):
            if verbose and warn:
                print(warn, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    _build_c_abi_program()
    return LIB


# A C99 program that runs a decode step through the C ABI alone (its GPU test
# checks it against the oracle); built beside the library.
C_ABI_SRC = os.path.join(ROOT, "tests", "c_abi_decode.c")
C_ABI_EXE = os.path.join(PKG, "c_abi_decode")


def _build_c_abi_program() -> None:
    if not os.path.exists(C_ABI_SRC) or shutil.which("gcc") is None:
        return
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = C_ABI_EXE + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(rocm, "include"), C_ABI_SRC,
           "-o", tmp, "-L" + PKG, "-l:libpagedkv.so", "-Wl,-rpath,$ORIGIN",
           "-L" + os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C ABI program failed to build:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, C_ABI_EXE)


if __name__ == "__main__":
    print(build(verbose=True))
