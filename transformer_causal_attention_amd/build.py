"""Compile the HIP sources into the in-tree shared library libattn.so (gfx950 only).

    python -m transformer_causal_attention_amd.build [-v]

Each source is compiled to an object under _build/ (in parallel), then linked.  hipcc
cross-compiles for gfx950 without a GPU present.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")

SOURCES = ["attn_api.cpp", "prep_kv.hip", "attn_fwd_bf16.hip", "attn_fwd_d256.hip", "attn_fwd_f32.hip", "attn_merge.hip",
           "attn_decode.hip", "attn_bwd.hip", "attn_bwd_d256.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
    f"-I{CSRC}",
]

# Per-source additions.  The backward kernels keep more than 256 registers live (one wave per
# SIMD): by default the compiler then places MFMA results in accumulation registers and moves
# them to the vector registers the softmax arithmetic reads, ~100 moves per step; with the
# vector-register form of the MFMA instructions it uses the accumulation registers only as
# storage for MFMA operands, which the MFMA reads directly.
EXTRA_FLAGS = {
    "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "attn_bwd_d256.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libattn.so")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose=False, jobs=4):
    """Compile every source and link libattn.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        _run([cc, *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
