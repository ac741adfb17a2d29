"""Builds libddl.so in-tree from csrc/ with hipcc for gfx950 (MI355X)."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libddl.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no packed fp32 VALU instructions in the device code.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
SOURCES = ["abi.cpp", "gemm.hip", "attn_prefill.hip", "rowops.hip", "decode.hip"]
# Per-source extras.  The attention kernel's MFMA accumulators are small and
# rescaled by VALU work every tile: keeping them in arch VGPRs (instead of
# AGPRs) saves the accvgpr moves.  The GEMMs need the AGPRs for their tiles.
EXTRA = {"attn_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if incremental and os.path.exists(obj):
        deps = [os.path.join(CSRC, src), os.path.join(CSRC, "common.h"),
                os.path.join(CSRC, "internal.h"), os.path.join(ROOT, "include", "ddl.h"), __file__]
        if os.path.getmtime(obj) > max(os.path.getmtime(d) for d in deps):
            return obj
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compiles every source (incremental=True: only those newer than their
    object file) and links libddl.so."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, incremental), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
    sys.exit(0)
