"""Builds libsubmconv.so in-tree with hipcc for gfx950.

Each HIP source is compiled to an object in parallel, then linked into one
shared library next to this file. Packed fp32 VALU instructions are disabled
for the device code.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsubmconv.so")
SOURCES = ["map_build.hip", "forward.hip", "backward.hip", "coord_ops.hip", "masked.hip",
           "staged.hip", "staged_wide.hip", "staged_bwd.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++20", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(os.path.dirname(HERE), "include")]
# keep MFMA accumulators in VGPRs: most kernels read and write them through
# LDS every step, which AGPRs would cost extra moves for
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# sources whose MFMA accumulators stay in registers for a whole unit (128 per
# lane) are built without it: the accumulators take the AGPRs, the operands
# the VGPRs
AGPR_SOURCES = {"staged_wide.hip", "staged_bwd.hip"}


def _compile(src, verbose):
    obj = os.path.join(CSRC, "_build", os.path.splitext(src)[0] + ".o")
    flags = FLAGS + ([] if src in AGPR_SOURCES else VGPR_FORM)
    cmd = [HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.join(CSRC, "_build"), exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
