"""Compile the HIP sources under csrc/ for gfx950 into libmoe.so (in-tree).

    python -m mixture_experts_layer_45_amd.build

Each .hip file is compiled on its own (in parallel) and the objects are linked
into one shared library exporting the C ABI of include/moe.h.  The routing
kernel is built without floating-point contraction so the sigmoid routing key
is exactly the written sequence of fp32 operations.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "route.hip", "permute.hip", "gemm.hip", "combine.hip", "backward.hip"]

COMMON = [
    "hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]
# route.hip: the selection keys must round exactly as specified (no contraction).
# gemm.hip: the one-lane tile claim must stay a plain atomic whose result is
# waited for only where it is used, not rewritten into a wave-wide reduction
# that waits (and drains the wave's in-flight loads) right after it.
PER_FILE = {"route.hip": ["-ffp-contract=off"],
            "gemm.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = COMMON + PER_FILE.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """The library with its host code (argument validation, workspace layout,
    launch set-up) built with AddressSanitizer and UndefinedBehaviorSanitizer
    (clang's runtime; the device code is built as usual): api.hip is compiled
    again with the sanitizers on the host pass only, the other objects are the
    ones build() made.  For the CPU sanitizer test."""
    objs = [os.path.join(BUILD, os.path.splitext(src)[0] + ".o") for src in SOURCES if src != "api.hip"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build() first: missing {missing}")
    obj = out + ".api.o"
    san = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    cmd = COMMON + san + ["-c", os.path.join(CSRC, "api.hip"), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on api.hip (sanitised):\n{r.stdout}\n{r.stderr}")
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address,undefined",
           "-shared-libsan", "-o", out, obj] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed (sanitised):\n{r.stdout}\n{r.stderr}")
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
