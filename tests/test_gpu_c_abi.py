"""The C ABI on a GPU from a plain C11 program (tests/c/abi_gpu_check.c),
without Python or torch in the process: hipMalloc'd buffers, the worked
example of four ranks by twenty int64 elements through ReduceScatter then
AllGather and through AllReduce for every schedule, and a rejected call that
leaves its outputs untouched.  The program is built in-tree with the library
(collective_reduction_amd._build.build_c_check) and runs as a child process.
"""

import os
import subprocess

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "abi_gpu_check")


def test_c_program_runs_every_schedule_on_the_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    assert os.path.exists(EXE), "tests/c/abi_gpu_check is not built: run __graft_entry__.build()"
    run = subprocess.run([EXE], capture_output=True, text=True, timeout=90)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.strip().splitlines()[-1] == "ok", run.stdout
