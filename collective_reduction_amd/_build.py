"""Build libccl_sim.so in-tree with hipcc for gfx950.

    python -m collective_reduction_amd._build [--extra-flag ...]

Each source is compiled to an object on its own thread, then the objects
are linked into the shared library.  The library is written next to this
file so that it travels with the source tree; the binding (``ccl_sim.py``)
loads it from there.
"""

import os
import shlex
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libccl_sim.so")
HOST_SOURCES = ["api.cpp", "model.cpp"]
KERNEL_SOURCES = ["kernels_direct.hip", "kernels_ring.hip", "kernels_recursive.hip", "kernels_misc.hip", "scratch.hip"]
SOURCES = [os.path.join(CSRC, s) for s in HOST_SOURCES + KERNEL_SOURCES]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 arithmetic.
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stdout}\n{proc.stderr}")
    noise = [ln for ln in proc.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)


C_CHECK = os.path.join(ROOT, "tests", "c", "abi_gpu_check.c")
C_CHECK_EXE = os.path.join(ROOT, "tests", "c", "abi_gpu_check")


def build_c_check(verbose=False):
    """The plain-C GPU check of the C ABI (tests/c/abi_gpu_check.c), linked
    against the in-tree library with a relative run path, so that it runs
    wherever the tree is copied.  Skipped without gcc."""
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None:
        return None
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = C_CHECK_EXE + ".tmp"
    _run([gcc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
          "-I", INCLUDE, "-I", os.path.join(rocm, "include"), C_CHECK, "-o", tmp,
          "-L", HERE, "-lccl_sim", "-Wl,-rpath,$ORIGIN/../../collective_reduction_amd",
          "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")], verbose)
    os.replace(tmp, C_CHECK_EXE)
    return C_CHECK_EXE


def build(extra_flags=(), output=LIB, verbose=False, jobs=None):
    """Compile every source and link ``output``; raises on failure."""
    jobs = jobs or min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with tempfile.TemporaryDirectory(prefix="ccl_sim_build_") as tmpdir:
        objects = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]
        cmds = [[HIPCC, *FLAGS, *extra_flags, "-x", "hip", "-c", src, "-o", obj] for src, obj in zip(SOURCES, objects)]
        with ThreadPoolExecutor(jobs) as pool:
            for f in [pool.submit(_run, cmd, verbose) for cmd in cmds]:
                f.result()
        tmp = output + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objects, "-o", tmp], verbose)
        os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
    print(build_c_check(verbose=True))
