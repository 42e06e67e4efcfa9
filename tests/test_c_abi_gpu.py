"""The C ABI used from C: tests/c/fa_abi_check.cpp calls libfa.so through include/fa.h alone
(hipMalloc'd buffers, forward, split forward, backward, error paths) and checks facts that hold
exactly for any correct attention. It runs as a child process."""

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "fa_abi_check")


def test_c_program_uses_the_abi():
    assert os.path.exists(EXE), f"{EXE} is not built (python -m exact_tiled_attention_23_amd.build)"
    print("running the C ABI check program", flush=True)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().splitlines()[-1] == "ok"
