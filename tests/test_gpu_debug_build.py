"""The MOE_DEBUG build (libmoe_debug.so: the grouped GEMM's operand loads range-checked by the
hardware, device index data validated on the host before each launch) computes exactly what
the release library computes on valid inputs (a bf16 layer forward and an MXFP8 training
step, bit for bit), and rejects corrupted index data (decreasing or out-of-range group
offsets, out-of-range gather indices and expert ids, repeated expert ids) with MOE_EINVAL
before launching anything. It runs in a child process with MOE_LIB set."""
import os
import subprocess
import sys

import numpy as np
import pytest

from tests.debug_build_run import run_layer, run_mx_step

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_LIB = os.path.join(ROOT, "dropless_mixture_experts_device_amd", "libmoe_debug.so")


def test_debug_build_matches_release_and_rejects_bad_index_data(tmp_path):
    if not os.path.exists(DEBUG_LIB):
        pytest.skip("libmoe_debug.so is not built (build(variant='debug'))")
    out = tmp_path / "debug.npz"
    env = dict(os.environ, MOE_LIB=DEBUG_LIB)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "debug_build_child.py"), str(out)],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    dbg = np.load(out)
    want = {}
    want.update(run_layer())
    want.update(run_mx_step())
    for n, v in want.items():
        np.testing.assert_array_equal(dbg[n], v, err_msg=n)
    assert sorted(dbg["rejected"].tolist()) == sorted([
        "offsets decreasing", "offsets past M", "gather index out of range", "expert id out of range",
        "expert id repeated"]), dbg["rejected"]
