"""GPU parity through the C ABI from a plain C program (tests/c_abi_parity.c):
hipMalloc'd buffers, the library's entry points, and the CPU oracle's C
functions as the reference -- no Python or torch between them."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_c_program_parity_through_the_abi():
    exe = os.path.join(ROOT, "tests", "c_abi_parity")
    if not os.path.exists(exe):
        pytest.fail("tests/c_abi_parity is not built: run __graft_entry__.build()")
    print("running tests/c_abi_parity (M, N, K = 384, 640, 512)", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
