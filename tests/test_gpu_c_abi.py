"""The library from plain C: a C program (tests/c_abi/c_check.c, built by the package's build
step) allocates device memory through the HIP runtime's C API, calls qknorm_fused,
normproj_fold_weight and normproj_deferred through include/qknorm.h, checks every output
against the fp64 oracle, and checks the status of a bad call. No Python runs in that process."""

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "c_check")


def test_plain_c_caller():
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() < 1:  # counting devices leaves HIP uninitialised here
        pytest.skip("no GPU")
    assert os.path.exists(EXE), "build first: python -c 'import __graft_entry__ as g; g.build()'"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=110)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi check ok" in r.stdout
