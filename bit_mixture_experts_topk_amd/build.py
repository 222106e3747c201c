"""Build libgnf4.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m bit_mixture_experts_topk_amd.build

Compiles every csrc/*.hip with hipcc in parallel and links one shared library
next to this file. Packed-FP32 instruction selection is disabled for all GPU
code (plain float code only).
"""

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libgnf4.so")
BUILD = os.path.join(HERE, "_build")
ARCH = "gfx950"


def revision():
    try:
        r = subprocess.run(["git", "-C", HERE, "rev-parse", "--short", "HEAD"],
                           capture_output=True, text=True, timeout=10)
        rev = r.stdout.strip() or "unknown"
        d = subprocess.run(["git", "-C", HERE, "status", "--porcelain", "--", "csrc"],
                           capture_output=True, text=True, timeout=10)
        return rev + ("+dirty" if d.stdout.strip() else "")
    except Exception:
        return "unknown"


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in VGPRs: the NF4 kernels scale every partial with VALU
            # FMAs, which cannot read accumulation registers
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-Wno-unused-command-line-argument",
            '-DGNF4_REVISION="%s"' % revision()]


def compile_one(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ["hipcc", "-c", src, "-o", obj] + flags()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = OUT + ".tmp"
    cmd = ["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
