"""Build the gfx950 shared library libgemm05.so in-tree with hipcc."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgemm05.so")
BUILD_DIR = os.path.join(HERE, "_build")

# Compiled in parallel: the ring kernel's instantiations are spread over
# several translation units.
SOURCES = ["g5_kernels.hip", "g5_ring_bt.hip", "g5_ring_at.hip", "g5_ring_epi.hip", "g5_fp8.hip", "g5_noalloc.hip", "g5_streamk.hip", "g5_act.hip",
           "g5_abi.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -packed-fp32-ops: keep the compiler from emitting packed FP32 VALU
# instructions (v_pk_*_f32); the hot loops here are matrix-core bound anyway.
# -amdgpu-mfma-vgpr-form=1: select the MFMA forms whose accumulators live in
# the unified VGPR file.  With the default heuristic the one-wave-per-SIMD
# kernels (192 accumulator registers per lane) got their accumulators split
# between AGPRs and VGPRs, with hundreds of copies per K slab and spills.
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-Wall", "-Wno-unused-function"]


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build_library(verbose=False):
    """Compile every source for gfx950 and link libgemm05.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
