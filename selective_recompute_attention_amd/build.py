"""Builds libsra.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m selective_recompute_attention_amd.build [-v] [--sanitize]

Every source is compiled on each call (objects go to _build/ at the repository root).

--sanitize builds a host-checked copy instead, _build/libsra_asan.so: the host pass of every source
(the C ABI's argument checks, planning and launch code) is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer, the device code as usual. It is for CPU runs of the ABI tests with the
sanitizer runtimes preloaded (SRA_LIB_PATH selects the library the binding loads):

    LD_PRELOAD=$(hipcc --print-file-name=libclang_rt.asan-x86_64.so) ASAN_OPTIONS=detect_leaks=0 \
        SRA_LIB_PATH=_build/libsra_asan.so python -m pytest tests/test_abi.py
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsra.so")
SOURCES = ["api.cpp", "rotate.hip", "anchors.hip", "score.hip", "score_f32.hip", "select.hip", "attn.hip",
           "stats.hip"]
ARCH = os.environ.get("SRA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         # packed fp32 ops stay off for every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # leading scalar and pointer kernel arguments arrive in SGPRs at wave launch (the code
         # object keeps a load prologue for firmware without the feature)
         "-mllvm", "-amdgpu-kernarg-preload-count=16",
         "-I", os.path.join(ROOT, "include")]


# host pass only: each option behind -Xarch_host, so no device code is built with a sanitizer
SANITIZE = [f for opt in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                          "-fno-omit-frame-pointer", "-g") for f in ("-Xarch_host", opt)]


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    obj_dir = os.path.join(OBJ, "asan") if sanitize else OBJ
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *(SANITIZE if sanitize else []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip() and verbose:
        print(out)
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    os.makedirs(os.path.join(OBJ, "asan") if sanitize else OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), SOURCES))
    lib = os.path.join(OBJ, "libsra_asan.so") if sanitize else LIB
    tmp = lib + ".tmp"
    # a sanitized library leaves the runtimes' symbols to the preloaded sanitizer runtime
    extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-shared-libasan"] if sanitize else []
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
