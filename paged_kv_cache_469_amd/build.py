"""Build the HIP library ``libpaged_attn.so`` in-tree for gfx950.

Every ``csrc/*.hip`` file is compiled with hipcc and every ``csrc/*.cpp``
file (host-only C++: the block manager) with g++, in parallel, and all are
linked into one shared library next to this file.  Each ``probes/*.hip``
(a standalone measurement program) becomes an executable beside its source.
Packed-FP32 instructions are switched off for all device code.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpaged_attn.so")
ARCH = os.environ.get("PAGED_ATTN_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
]


# Extra flags per source.  The prefill kernel keeps two waves per SIMD at the
# 256-register limit; the iterative-ILP machine scheduler issues its LDS
# operand reads several MFMAs ahead instead of one at a time.  Its scores are
# never NaN (unused rows come from a zero line), so fmaxf needs no NaN
# quieting of its operands (-fno-honor-nans; infinities are still honoured).
# Its one-lane atomics stay plain atomics: the atomic optimizer would wait
# for the returned value right after the atomic, which stalls the wave.
PER_FILE = {
    "prefill.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp", "-fno-honor-nans",
                    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
}


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]


def _compile(src):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    if src.endswith(".cpp"):
        cmd = [shutil.which("g++") or "g++", *HOST_FLAGS, "-c", src, "-o", obj]
    else:
        cmd = [_hipcc(), *FLAGS, *PER_FILE.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


PROBES = os.path.join(HERE, "probes")


def _probe(src):
    """A measurement probe: one standalone executable per probes/*.hip."""
    exe = src[:-len(".hip")]
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return exe


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    probes = sorted(os.path.join(PROBES, f) for f in os.listdir(PROBES) if f.endswith(".hip")) \
        if os.path.isdir(PROBES) else []
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probes))) as ex:
        probe_jobs = [ex.submit(_probe, p) for p in probes]
        objs = list(ex.map(_compile, srcs))
        for j in probe_jobs:
            j.result()
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
