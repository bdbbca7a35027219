"""Build liblamp.so (gfx950 only) in-tree with hipcc.

Each translation unit is compiled to an object file in parallel, then linked
into ``mixed_precision_tiled_amd/liblamp.so``.  The sustained-MFMA probe of
the measurement harness is linked on its own into
``mixed_precision_tiled_amd/libmfma_probe.so``.  Always rebuilds.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liblamp.so")
PROBE_SRC = os.path.join(HERE, "probe", "mfma_sustained.hip")
PROBE_OUT = os.path.join(HERE, "libmfma_probe.so")
BUILD = os.path.join(HERE, "_build")

SOURCES = ["lamp_api.cpp", "quant_mask.hip", "attn_d64.hip", "attn_d128.hip", "attn_d256.hip",
           "decode.hip"]

# Per-unit flags.  Head dim 256 runs one wave per SIMD with 512 registers;
# there the compiler would put every MFMA accumulator in AGPRs, and the
# logits would travel AGPR -> VGPR -> AGPR between the products and the
# softmax.  The VGPR form keeps them in VGPRs (AGPRs still take the
# overflow).  With a single wave per SIMD nothing hides the latency of one
# instruction behind another wave's: the ILP-oriented machine scheduler
# spreads dependent instructions further apart.
UNIT_FLAGS = {"attn_d256.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true",
                                "-mllvm", "--amdgpu-sched-strategy=iterative-ilp"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed fp32 VALU forms are switched off for every HIP translation unit
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        _run([HIPCC, *FLAGS, *UNIT_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    def compile_probe():
        tmp = PROBE_OUT + ".tmp"
        _run([HIPCC, *FLAGS, "-shared", PROBE_SRC, "-o", tmp])
        os.replace(tmp, PROBE_OUT)

    with ThreadPoolExecutor(jobs) as ex:
        probe = ex.submit(compile_probe)
        objs = list(ex.map(compile_one, SOURCES))
        probe.result()
    tmp = OUT + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
