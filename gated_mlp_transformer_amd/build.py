"""Build libmoeffn.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python gated_mlp_transformer_amd/build.py

Compiles every ``csrc/*.hip`` to an object under ``_build/`` and links the
shared library next to this file. hipcc cross-compiles for gfx950, so no GPU
is needed to build.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoeffn.so")
ARCH = "gfx950"

# Packed fp32 VALU ops are kept off: hipcc -O3 would otherwise form
# v_pk_{add,mul,fma}_f32 from scalar or float2 code by itself.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoeffn.so)")


# Per-source flags. The fp8 GEMMs scale each 128-deep partial sum with
# fp32 FMAs; with the MFMA results in VGPRs (not AGPRs) those FMAs read them
# directly instead of through one v_accvgpr_read per element (fp8-activation
# prefill: gate/up 332 -> 317 us, down 201 -> 183 us). The tiled fp8-weight
# kernel (gemm_w8.hip) is left out: with the option it spills ~130 VGPRs into
# AGPRs and runs 1.45x slower.
FILE_FLAGS = {
    "gemm_a8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "gemm_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = FILE_FLAGS.get(os.path.basename(src), [])
    cmd = [hipcc(), *HIP_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile and link; always rebuilds. Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           "-Wl,-Bsymbolic"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", flush=True)
    return LIB


if __name__ == "__main__":
    build()
