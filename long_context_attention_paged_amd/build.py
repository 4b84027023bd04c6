"""Build libkvattn.so in-tree with hipcc for gfx950.

Every translation unit is compiled to an object under _build/ (in parallel),
then linked into long_context_attention_paged_amd/libkvattn.so. Packed fp32
vector instructions are disabled for all device code.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvattn.so")
SOURCES = ["api.hip", "quantize.hip", "select.hip", "merge.hip", "decode.hip", "prefill.hip",
           "gather.hip", "rotate.hip"]
# The decode and prefill kernels keep their 64-128 loop-carried accumulators
# in VGPRs next to LDS-staged operands; without this the allocator splits them
# between VGPRs and AGPRs and copies every accumulator on each loop iteration.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
# The prefill kernel's operands are finite by contract (include/kvattn.h):
# without NaN semantics its row maxima need no quieting of each product,
# which takes ~1% off a kernel whose vector work sits on the critical path.
EXTRA_FLAGS = {"decode.hip": _VGPR_FORM, "prefill.hip": _VGPR_FORM + ["-fno-honor-nans"]}
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libkvattn")
    return exe


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
