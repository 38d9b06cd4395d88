"""Compile libgrz.so (HIP, gfx950) in-tree with hipcc.

``python -m gradient_reduce_zero_amd.build`` or ``build()``.  The flags matter
for the numerics: ``-ffp-contract=off`` keeps every multiply and add rounded
on its own and ``-fhip-fp32-correctly-rounded-divide-sqrt`` keeps fp32
division and square root IEEE-exact; packed fp32 instructions are switched off.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "grz.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgrz.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(out=LIB, extra=(), verbose=False):
    """Compile the library to ``out`` (atomically replaced) and return its path."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra, f"-I{INCLUDE}", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
