"""The binding must work when a program calls it before importing torch.
torch ships its own HIP runtime under the system runtime's soname, so a
process that loaded the library (and with it the system runtime) first would
hold two runtimes, and every launch on torch's streams failed.  The child
process below loads the library before anything imports torch, quantizes a
seeded tensor, and the codes and scales must equal the oracle's."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from blockwise_fp8_linear_amd import synth
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
assert "torch" not in sys.modules
import blockwise_fp8_linear_amd as fb
assert "torch" not in sys.modules
fb.load_library()
import numpy as np
import torch
x = np.load(sys.argv[2])
xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
q, s = fb.fp8_quantize_rowgroup(xt)
torch.cuda.synchronize()
np.save(sys.argv[3], q.cpu().numpy())
np.save(sys.argv[4], s.cpu().numpy())
"""


def test_library_loaded_before_torch(tmp_path):
    require_gpu()
    x = synth.normal_bf16((256, 512), 1.0, 71, 0)
    xin, qout, sout = tmp_path / "x.npy", tmp_path / "q.npy", tmp_path / "s.npy"
    np.save(xin, x)
    print(f"[load order] child quantizes {x.shape}", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, str(xin), str(qout), str(sout)], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    q0, s0 = oracle.quantize_rowgroup(x)
    assert np.array_equal(np.load(sout), s0)
    assert np.array_equal(np.load(qout), q0)
