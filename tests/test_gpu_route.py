"""moe_route on the GPU vs the oracle: exact keys and selections on exactly representable
inputs (every tie broken the same way), tolerance-bound keys and margin-checked selections
on the seeded workloads at their full sizes."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as O
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    from dropless_mixture_experts_device_amd import _lib
    return _lib


def _run(L, x, w, bias, k, score, want_keys=True):
    T, E = x.shape[0], w.shape[0]
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    wt = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    keys = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda") if want_keys else None
    nb = L.moe_workspace_bytes(L.MOE_OP_ROUTE, T, x.shape[1], E, k, 0)
    ws = torch.empty((max(nb, 256),), dtype=torch.uint8, device="cuda")
    L.moe_route(x, w, bias, k, score, idx, wt, keys, workspace=ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), wt.cpu().numpy().astype(np.float64), None if keys is None else keys.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,d,E,k,score", [(300, 512, 8, 2, "softmax"), (77, 256, 64, 8, "sigmoid"),
                                           (130, 1024, 256, 8, "sigmoid"), (33, 64, 128, 1, "softmax"),
                                           (5, 128, 16, 16, "softmax"), (64, 7168, 256, 8, "sigmoid"),
                                           (1000, 2048, 128, 8, "softmax"), (777, 7168, 256, 8, "sigmoid"),
                                           (300, 1024, 64, 4, "sigmoid")])
def test_route_exact_inputs_bit_exact(L, dtype, T, d, E, k, score):
    # small integers times powers of two: every partial sum is exact in fp32, so the GPU's
    # keys must equal the oracle's bit for bit and many keys tie (pins the tie-break)
    x = mi.integer_valued((T, d), -2, 2, 0, T + d)
    w = mi.integer_valued((E, d), -1, 1, -4, E + k)
    b = mi.integer_valued((E,), -4, 4, -3, 7)
    sc = L.MOE_SOFTMAX if score == "softmax" else L.MOE_SIGMOID
    idx, wt, keys = _run(L, dev(x, dtype), dev(w, dtype), torch.from_numpy(b).cuda(), k, sc)
    want_keys = O.router_keys(x, w, b)
    np.testing.assert_array_equal(keys, want_keys)
    want_idx = O.select_topk(want_keys, k)
    np.testing.assert_array_equal(idx, want_idx)
    np.testing.assert_allclose(wt, O.topk_weights(want_keys, want_idx, score), rtol=0, atol=2e-6)


@pytest.mark.parametrize("name", ["tiny", "small_softmax", "small_sigmoid", "mixtral", "qwen3", "dsv3"])
def test_route_workloads(L, name):
    w = mi.WORKLOADS[name]
    dt =torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x = torch.empty((w.T, w.d), dtype=dt, device="cuda")
    mi.randn_torch(w.seed, mi.X, 0, w.T, w.d, w.sigma_x, w.dtype, "cuda", out=x)
    wr = torch.empty((w.E, w.d), dtype=dt, device="cuda")
    mi.randn_torch(w.seed, mi.W_ROUTER, 0, w.E, w.d, w.sigma_w, w.dtype, "cuda", out=wr)
    b = mi.expert_bias(w)
    sc = L.MOE_SOFTMAX if w.score == "softmax" else L.MOE_SIGMOID
    idx, wt, keys = _run(L, x, wr, None if b is None else torch.from_numpy(b).cuda(), w.k, sc)
    ok_keys = O.router_keys(mi.x_np(w), mi.w_router_np(w), b).astype(np.float64)
    dk = np.abs(keys.astype(np.float64) - ok_keys)
    assert dk.max() <= 1e-4, dk.max()
    margin = 2 * dk.max()
    o_idx = O.select_topk(ok_keys, w.k)
    srt = -np.sort(-ok_keys, axis=1)
    gap = srt[:, w.k - 1] - srt[:, w.k] if w.k < w.E else np.full(w.T, np.inf)
    clear = gap > margin
    np.testing.assert_array_equal(idx[clear], o_idx[clear])
    # tokens too close to call: the GPU's choice must still be a valid top-k within the margin
    for t in np.flatnonzero(~clear):
        chosen = ok_keys[t, idx[t]]
        rest = np.delete(ok_keys[t], idx[t])
        assert len(set(idx[t].tolist())) == w.k
        assert chosen.min() >= rest.max() - margin
    ow = O.topk_weights(ok_keys, idx, w.score)
    np.testing.assert_allclose(wt, ow, rtol=0, atol=2e-6 + 2 * float(dk.max()))
    np.testing.assert_allclose(wt.sum(1), 1.0, atol=1e-6)
    print(f"{name}: max|dkey| {dk.max():.2e}, ambiguous tokens {int((~clear).sum())}")
