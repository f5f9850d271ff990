"""Build libccl_sim.so in-tree with hipcc for gfx950.

    python -m collective_reduction_amd._build [--extra-flag ...]

The library is written next to this file so that it travels with the source
tree; the binding (``ccl_sim.py``) loads it from there.
"""

import os
import shlex
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libccl_sim.so")
SOURCES = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "model.cpp"), os.path.join(CSRC, "kernels.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 arithmetic.
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def build(extra_flags=(), output=LIB, verbose=False):
    """Compile every HIP source into ``output``; raises on failure."""
    tmp = output + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra_flags, "-x", "hip", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stdout}\n{proc.stderr}")
    noise = [ln for ln in proc.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
