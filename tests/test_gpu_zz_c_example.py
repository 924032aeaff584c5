"""The C ABI from C++: the example program built next to the library calls it with hipMalloc'd
buffers and no Python in the path (validation contract, ring order independence)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "long_context_exact_blockattn_amd", "abi_example")


def test_c_caller_validation_and_ring_order_independence():
    assert os.path.exists(EXE), f"{EXE} is missing: run __graft_entry__.build() first"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("abi_example ok")
