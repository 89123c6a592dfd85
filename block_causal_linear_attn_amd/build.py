"""Build liblinscan.so in-tree with hipcc for gfx950.

    python -m block_causal_linear_attn_amd.build

compiles every source under csrc/ into block_causal_linear_attn_amd/liblinscan.so.
Packed-fp32 instruction selection is switched off for the device code; the
host pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "liblinscan.so")
ARCH = os.environ.get("LINSCAN_ARCH", "gfx950")


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip"))) + \
        sorted(glob.glob(os.path.join(HERE, "csrc", "*.cpp")))


FLAGS = ["-O3", "-std=c++17", "--offload-arch=" + ARCH, "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; drop that line only
    err = "\n".join(l for l in res.stderr.splitlines() if NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError("%s failed (%d):\n%s" % (" ".join(cmd), res.returncode, err))
    return err


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile each source to an object in parallel, then link the shared library."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    cmds = [["hipcc"] + FLAGS + ["-I" + os.path.join(ROOT, "include"), "-c", s, "-o", o]
            for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        for cmd, err in zip(cmds, ex.map(_run, cmds)):
            if verbose:
                print(" ".join(cmd), flush=True)
                if err.strip():
                    print(err, file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run(["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
