"""The library's device calls work when the package is imported before torch:
a fresh interpreter imports the package first, then runs one step of the
tiny layer and checks it against the oracle (routing certified, outputs
within 2e-3 of max|y|)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_STEP = r"""
import sys
sys.path[:0] = [sys.argv[1], sys.argv[1] + "/tests"]
import sparse_moe_decode_router_amd as moe   # before anything imports torch
import numpy as np
import torch
import moe_synth as ms
from gpu_support import DeviceLayer, certify_routing, assert_close_y

L = DeviceLayer(ms.CONFIGS["tiny"])
xb, x = L.x(0, 4)
y, idx, w, s = moe.moe_layer_forward(L.layer, x, path=moe.MOE_PATH_DECODE)
torch.cuda.synchronize()
idx = idx.cpu().numpy()
depth = moe.moe_router_sum_depth(xb.shape[0], L.cfg.d, L.cfg.E)
namb, _ = certify_routing(xb, L.Wr_np, L.bias_np, L.cfg.k, idx, depth)
ref = L.oracle(xb, idx=idx if namb else None)
assert np.array_equal(idx, ref["idx"])
print("rel", assert_close_y(y.cpu().numpy(), ref["y"]), flush=True)
"""


def test_device_calls_with_the_package_imported_before_torch():
    r = subprocess.run([sys.executable, "-c", _STEP, ROOT], capture_output=True, text=True, timeout=100)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.split()[0] == "rel", r.stdout
