"""Build libmustafar.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmustafar.so")
# the slowest translation units first, so that the parallel build finishes early
SOURCES = ["decode_sparse_mfma_g4.hip", "decode_sparse_mfma_g8.hip", "decode_sparse_mfma_g2.hip",
           "decode_sparse_mfma_g1.hip", "decode_24.hip", "decode_sparse.hip", "decode_dense.hip",
           "decode_sparse_mfma.hip", "api.hip", "prune.hip", "util.hip"]
ARCH = os.environ.get("MUSTAFAR_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
    # keep the compiler from emitting packed-fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# Matrix-core kernels: MFMA accumulators in ordinary VGPRs, so the vector code
# that rescales them needs no copies to and from the accumulation registers.
FILE_FLAGS = {
    **{f"decode_sparse_mfma_g{g}.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"] for g in (1, 2, 4, 8)},
    "decode_24.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "decode_dense.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = ["hipcc", *FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
