"""The C ABI from C++ alone: tests/c_abi/fckl_c_driver (built by __graft_entry__.build())
allocates with hipMalloc and calls include/fckl.h directly, with no Python binding and
no torch, and checks its results (see the driver's header)."""
import os
import subprocess

import pytest
import torch

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "fckl_c_driver")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def test_c_abi_driver():
    assert os.path.exists(EXE), "build the driver first (__graft_entry__.build())"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout.strip())
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "c abi driver ok" in r.stdout
