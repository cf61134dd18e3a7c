"""Builds libidx.so (the HIP kernels and the C ABI of include/idx.h) in-tree for gfx950.

    python -m sparse_attention_indexer_02_amd.build      (or __graft_entry__.build())

Each .hip source is compiled to an object under _build/ in parallel, then linked into
sparse_attention_indexer_02_amd/libidx.so. Always recompiles.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libidx.so")
SOURCES = ["abi.hip", "score.hip", "score_f8f8.hip", "score_bb128.hip", "score_bb64.hip", "score_bb32_b8.hip",
           "score_f32_f32_d128.hip", "score_f32_bf16_d128.hip", "score_f32_fp8_d128.hip",
           "score_f32_f32_d32_64.hip", "score_f32_bf16_d32_64.hip", "score_f32_fp8_d32_64.hip",
           "block_refine.hip", "decode.hip", "topk.hip", "prep.hip", "latent.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed-fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]
# Per-source flags. decode.hip keeps its query fragments in the accumulation registers (they are
# only MFMA operands); this makes the MFMAs write their results to ordinary vector registers, so
# the epilogue reads them without copies.
EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(os.cpu_count() or 8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
