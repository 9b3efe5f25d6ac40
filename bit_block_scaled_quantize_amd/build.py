"""Build libnvfp4.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Flags that matter for correctness:
  -ffp-contract=off            every a*b+c rounds twice, as the format's
                               definition is written (no FMA contraction);
  -fhip-fp32-correctly-rounded-divide-sqrt
                               the per-block division and reciprocal are
                               correctly rounded binary32 operations;
  -fno-gpu-flush-denormals-to-zero
                               binary32 subnormals are kept;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                               no packed FP32 instructions are generated.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libnvfp4.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["quantize.hip", "gemm.hip", "mx.hip", "mx_gemm.hip", "nvfp4_api.hip"]
ARCH = os.environ.get("NVFP4_OFFLOAD_ARCH", "gfx950")


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the NVFP4 HIP library cannot be built")
    return exe


def flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
            "-fno-gpu-flush-denormals-to-zero",
            # loops marked for full unrolling stay unrolled even when the body
            # is large (a rolled loop would index register arrays dynamically)
            "-mllvm", "-pragma-unroll-threshold=262144",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-I", CSRC, "-I", INCLUDE]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False):
    """Compile every source and link libnvfp4.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
