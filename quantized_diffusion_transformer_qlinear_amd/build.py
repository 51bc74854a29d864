"""Build the qlinear HIP library for gfx950 (in-tree: libaria_qlinear.so next
to this file).  Every .hip source under csrc/ is compiled with hipcc to an
object in _build/, then linked into one shared library exporting the C-ABI of
include/aria_qlinear.h."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libaria_qlinear.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off (plain fp32 code is emitted instead)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division: the quantizers depend on a correctly rounded quotient
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
]


# per-source additions: MFMA accumulators in ordinary VGPRs (the VGPR form of
# MFMA).  The attention kernel does VALU work (softmax, rescaling) on its MFMA
# results every key block, which accumulation registers would first have to
# copy out; the 4-wave GEMM tiles otherwise get accumulation registers on top
# of their VGPRs and drop to one wave per SIMD.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA = {"attention.hip": VGPR_FORM, "gemm_tiled.hip": VGPR_FORM}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")
    extra = EXTRA.get(os.path.basename(src), [])
    r = subprocess.run([HIPCC, *FLAGS, *extra, "-c", src, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=jobs or min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
