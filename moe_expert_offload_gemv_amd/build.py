"""Build libmoe_offload.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m moe_expert_offload_gemv_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libmoe_offload.so")
OBJDIR = os.path.join(ROOT, "_build", "moe_offload")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

SOURCES = ["route.hip", "decode.hip", "decode_layer.hip", "prefill_kernels.hip", "measure.hip", "step_copy.hip", "scratch.hip", "grouped_mfma.hip",
           "runtime.cpp", "prefill.cpp", "host_experts.cpp"]
# plain C++ with no HIP in it (x86 vector code chosen at run time), built by the host compiler
HOST_ONLY = {"host_experts.cpp"}
CXX = os.environ.get("CXX_HOST", "g++")
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    # no packed fp32 instructions in any device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


# per-file code generation options: the grouped MFMA kernels scale each MFMA
# result in VALU right away, so their results go to VGPRs (the AGPR form
# would add a v_accvgpr_read per result element)
EXTRA_FLAGS = {"grouped_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJDIR, src + ".o")
    if src in HOST_ONLY:
        cmd = [CXX, *HOST_FLAGS, "-c", path, "-o", obj]
    else:
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), *lang, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
