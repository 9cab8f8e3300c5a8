"""moe_permute on the GPU vs the oracle: offsets, row_of, src_token and the gathered rows
must match bit for bit, from the oracle's own routing of each workload and from edge cases."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as O
from tests.gpu_util import bits, dev, dev_i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    from dropless_mixture_experts_device_amd import _lib
    return _lib


def _gpu_permute(L, x_dev, topk_idx, E, shared, gather=True):
    T, k = topk_idx.shape
    rows = T * k + (T if shared else 0)
    d = x_dev.shape[1]
    off = torch.full((E + 2,), -9, dtype=torch.int32, device="cuda")
    ro = torch.full((T, k), -9, dtype=torch.int32, device="cuda")
    src = torch.full((rows,), -9, dtype=torch.int32, device="cuda")
    xp = torch.full((rows, d), float("nan"), dtype=x_dev.dtype, device="cuda") if gather else None
    ws = torch.empty((L.moe_workspace_bytes(L.MOE_OP_PERMUTE, T, d, E, k, 0),), dtype=torch.uint8, device="cuda")
    L.moe_permute(x_dev if gather else None, dev_i32(topk_idx), E, shared, off, ro, src, xp, ws, d=d,
                  dtype=L._dtype(x_dev))
    torch.cuda.synchronize()
    n_off = E + (2 if shared else 1)
    return off[:n_off].cpu().numpy(), ro.cpu().numpy(), src.cpu().numpy(), xp


def _check(L, x, topk_idx, E, shared, dtype="bf16", gather=True):
    x_dev = dev(x, dtype)
    off, ro, src, xp = _gpu_permute(L, x_dev, topk_idx, E, shared, gather)
    w_off, w_ro, w_src = O.permutation(topk_idx, E, x.shape[0] if shared else 0)
    np.testing.assert_array_equal(off, w_off)
    np.testing.assert_array_equal(ro, w_ro)
    np.testing.assert_array_equal(src, w_src)
    if gather:
        want = dev(O.gather_rows(x, w_src), dtype)
        np.testing.assert_array_equal(bits(xp), bits(want))


@pytest.mark.parametrize("name", ["tiny", "small_softmax", "small_sigmoid", "mixtral", "qwen3", "dsv3"])
def test_permute_workload_routing(L, name):
    w = mi.WORKLOADS[name]
    x = mi.x_np(w)
    idx, _, _ = O.route(x, mi.w_router_np(w), mi.expert_bias(w), w.k, w.score)
    _check(L, x, idx, w.E, bool(w.shared_f), w.dtype)


def _topk(T, E, k, seed, hot=None):
    g = np.random.Generator(np.random.PCG64(seed))
    out = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else np.zeros((0, k), np.int32)
    if hot is not None:
        for t in range(T):
            row = [hot] + [e for e in out[t] if e != hot][:k - 1]
            out[t] = row
    return out


@pytest.mark.parametrize("T,E,k,shared,gather,hot", [
    (1, 1, 1, False, True, None),          # a single pair
    (1, 4, 4, True, True, None),
    (63, 3, 2, False, True, None),
    (1025, 16, 4, True, True, None),       # two 1024-token tiles, ragged tail
    (2049, 64, 8, False, False, None),     # indices only
    (3000, 8, 1, False, True, 5),          # one expert takes every token, the rest are empty
    (4096, 256, 8, True, False, 0),
])
def test_permute_edge_cases(L, T, E, k, shared, gather, hot):
    x = mi.randn_np(99, mi.X, 0, T, 64, 1.0, "bf16")
    _check(L, x, _topk(T, E, k, T + E, hot), E, shared, "bf16", gather)


def test_permute_fp32_rows(L):
    x = mi.randn_np(5, mi.X, 0, 500, 40, 1.0, "f32")
    _check(L, x, _topk(500, 12, 3, 1), 12, True, "f32", True)
