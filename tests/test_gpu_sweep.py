"""The whole layer forward over a seeded sweep of shapes (moe_inputs.fuzz_workloads: E from 1
to 256, k from 1 to min(8, E), T from 1 to 9000, softmax and sigmoid, shared expert or not,
Zipf skew or forced empty groups, bf16 and fp32) against the oracle.

Routing is checked against the oracle's keys with a margin (a token whose k-th and (k+1)-th
keys are closer than the projection's rounding may pick either); everything after it runs
on the GPU's own routing and must match the oracle's permutation bit for bit and its H, Y
and output within the storage dtype's gate. Experts the inputs make unselectable must come
back as empty groups."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as O
from tests.gpu_util import DeviceWorkload, assert_close, host

pytestmark = pytest.mark.gpu

SWEEP = mi.fuzz_workloads()


@pytest.fixture(scope="module")
def LY():
    from dropless_mixture_experts_device_amd import _lib, layer
    return _lib, layer


@pytest.mark.parametrize("w", SWEEP, ids=[w.name for w in SWEEP])
def test_layer_sweep(LY, w):
    L, layer = LY
    print(f"{w.name}: T={w.T} d={w.d} f={w.f} E={w.E} k={w.k} {w.dtype} {w.score} bias={w.bias} "
          f"shared={w.shared_f}", flush=True)
    dw = DeviceWorkload(w)
    s = layer.LayerShape(T=w.T, d=w.d, f=w.f, E=w.E, k=w.k, shared=bool(w.shared_f),
                         score=L.MOE_SOFTMAX if w.score == "softmax" else L.MOE_SIGMOID,
                         dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    b = layer.LayerBuffers(s, "cuda")
    keys = torch.full((w.T, w.E), float("nan"), dtype=torch.float32, device="cuda")
    layer.route(dw.x, dw.w_router, dw.bias, s, b, keys_out=keys)
    layer.permute(dw.x, s, b)
    layer.experts(dw.x, dw.w_gu, dw.w_down, s, b)
    layer.combine(s, b)
    torch.cuda.synchronize()

    # routing: keys within the projection's rounding, selections margin-checked
    x = mi.x_np(w).astype(np.float64)
    bias = mi.expert_bias(w)
    ok_keys = O.router_keys(x, mi.w_router_np(w), bias)
    gk = host(keys)
    dk = np.abs(gk - ok_keys) / np.maximum(1.0, np.abs(ok_keys))
    assert dk.max() <= (1e-4 if w.dtype == "bf16" else 1e-5), dk.max()
    idx = b.topk_idx.cpu().numpy()
    wt = b.topk_w.cpu().numpy().astype(np.float64)
    margin = 2 * float(np.max(np.abs(gk - ok_keys))) + 1e-12
    o_idx = O.select_topk(ok_keys, w.k)
    srt = -np.sort(-ok_keys, axis=1)
    gap = srt[:, w.k - 1] - srt[:, w.k] if w.k < w.E else np.full(w.T, np.inf)
    clear = gap > margin
    np.testing.assert_array_equal(idx[clear], o_idx[clear])
    for t in np.flatnonzero(~clear):
        assert len(set(idx[t].tolist())) == w.k
        assert ok_keys[t, idx[t]].min() >= np.delete(ok_keys[t], idx[t]).max() - margin
    np.testing.assert_allclose(wt, O.topk_weights(ok_keys, idx, w.score), rtol=0, atol=2e-6 + 2 * margin)

    # the rest on the GPU's routing
    rnd = O.round_bf16 if w.dtype == "bf16" else O.round_f32
    ref = O.layer_forward(x, None, None, w.k, w.score, lambda e: mi.w_gate_up_np(w, e),
                          lambda e: mi.w_down_np(w, e), w.E, shared=bool(w.shared_f), rnd=rnd, topk=(idx, wt))
    off = b.offsets.cpu().numpy()
    np.testing.assert_array_equal(off, ref["offsets"])
    np.testing.assert_array_equal(b.row_of.cpu().numpy(), ref["row_of"])
    np.testing.assert_array_equal(b.src_token.cpu().numpy(), ref["src_token"])
    if w.bias is not None and w.bias[0] == "dead":
        dead = np.flatnonzero(bias < -1.0)
        assert np.all(np.diff(off)[dead] == 0), "an unselectable expert received rows"
    R = int(off[-1])
    assert_close(host(b.H[:R]), ref["H"], w.dtype, "H")
    assert_close(host(b.Y[:R]), ref["Y"], w.dtype, "Y")
    mx, mean = assert_close(host(b.out), ref["out"], w.dtype, "out")
    print(f"  groups {len(off) - 1}, empty {int((np.diff(off) == 0).sum())}, ambiguous tokens "
          f"{int((~clear).sum())}, out max rel {mx:.2e} mean rel {mean:.2e}")
