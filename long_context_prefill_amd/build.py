"""Build libminf.so (all HIP sources under csrc/) for gfx950 with hipcc.

The library is built in-tree, next to this file, so that it travels with the
source tree.  Usage: python -m long_context_prefill_amd.build [--jobs N]
"""
import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libminf.so")
OBJDIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the kernels never produce NaN (excluded pairs are -inf, and every
    # -inf - -inf is guarded), so max/min need no NaN quieting; infinities
    # are still honoured
    "-fno-honor-nans",
    "-Wno-unused-result", "-Wno-unused-command-line-argument",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# Per-file flags.  attn_bf16.hip takes the next work item's queue ticket
# with one lane's atomic during the current item and uses the value only at
# the item's end; the compiler's atomic optimizer would turn that atomic into
# a wave-wide reduction whose result is waited for at once.
FILE_FLAGS = {"attn_bf16.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(cc, src, extra):
    obj = os.path.join(OBJDIR, os.path.basename(src)[:-4] + ".o")
    cmd = [cc] + FLAGS + FILE_FLAGS.get(os.path.basename(src), []) + extra + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs=None, extra=None, verbose=False):
    cc = hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    extra = list(extra or [])
    srcs = sources()
    with ThreadPoolExecutor(jobs or min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(cc, s, extra), srcs))
    tmp = OUT + ".tmp"
    cmd = [cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args()
    build(a.jobs, verbose=True)
    sys.exit(0)
