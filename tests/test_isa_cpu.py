"""Properties of the gfx950 code the kernels compile to (no GPU needed).

Each kernel source is compiled to device assembly with the library's own
flags, and the assembly must hold:

* no packed float32 arithmetic: the build turns the feature off, and none
  is written by hand;
* no scalar-cache writes of any kind (scalar stores, scalar atomics, or
  the scalar cache's write-back and discard): every store goes through the
  vector memory path;
* no scratch (private) memory: nothing spills, so no kernel needs a
  per-lane stack.
"""

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from collective_reduction_amd import _build

SCALAR_WRITE = re.compile(r"^\s*s_(buffer_)?(store|atomic)\w*|^\s*s_dcache_(wb|discard)\w*", re.M)
PACKED_FP32 = re.compile(r"^\s*v_pk_(add|mul|fma)_f32\b", re.M)
SCRATCH_USE = re.compile(r"^\s*scratch_\w+", re.M)
PRIVATE_SIZE = re.compile(r"\.private_segment_fixed_size:\s*(\d+)")


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    if not os.path.exists(_build.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("no hipcc")
    out = tmp_path_factory.mktemp("isa")
    flags = [f for f in _build.FLAGS if f not in ("-fPIC",)]

    def compile_one(name):
        src = os.path.join(_build.CSRC, name)
        dst = str(out / (name + ".s"))
        proc = subprocess.run([_build.HIPCC, *flags, "-x", "hip", "--cuda-device-only", "-S", src, "-o", dst],
                              capture_output=True, text=True)
        assert proc.returncode == 0, proc.stderr[-2000:]
        return name, open(dst).read()

    with ThreadPoolExecutor(len(_build.KERNEL_SOURCES)) as pool:
        return dict(pool.map(compile_one, _build.KERNEL_SOURCES))


@pytest.mark.parametrize("name", _build.KERNEL_SOURCES)
def test_kernel_assembly_properties(assembly, name):
    text = assembly[name]
    assert ".amdhsa_kernel" in text or ".amdgpu_hsa_kernel" in text or "amdhsa.kernels" in text
    assert not SCALAR_WRITE.search(text), SCALAR_WRITE.search(text).group(0)
    assert not PACKED_FP32.search(text), PACKED_FP32.search(text).group(0)
    assert not SCRATCH_USE.search(text), SCRATCH_USE.search(text).group(0)
    sizes = [int(v) for v in PRIVATE_SIZE.findall(text)]
    if name == "scratch.hip":
        # device data only (the no-allocation entry point's array), no kernel
        assert not sizes
        return
    assert sizes and max(sizes) == 0, f"private segment sizes {sorted(set(sizes))}"
