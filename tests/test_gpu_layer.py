"""The whole layer forward on the GPU (route -> permute -> grouped SwiGLU MLP -> combine)
vs the oracle, HIP-graph replay with new routings, and run-to-run determinism."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as O
from tests.gpu_util import DeviceWorkload, assert_close, bits, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def LY():
    from dropless_mixture_experts_device_amd import _lib, layer
    return _lib, layer


def _shape(L, layer, w):
    return layer.LayerShape(T=w.T, d=w.d, f=w.f, E=w.E, k=w.k, shared=bool(w.shared_f),
                            score=L.MOE_SOFTMAX if w.score == "softmax" else L.MOE_SIGMOID,
                            dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32)


def _oracle(w):
    rnd = O.round_bf16 if w.dtype == "bf16" else O.round_f32
    return O.layer_forward(mi.x_np(w), mi.w_router_np(w), mi.expert_bias(w), w.k, w.score,
                           lambda e: mi.w_gate_up_np(w, e), lambda e: mi.w_down_np(w, e), w.E,
                           shared=bool(w.shared_f), rnd=rnd)


@pytest.mark.parametrize("name", ["tiny", "small_softmax", "small_sigmoid"])
@pytest.mark.parametrize("fused", [True, False])
def test_layer_forward_small(LY, name, fused):
    L, layer = LY
    w = mi.WORKLOADS[name]
    dw = DeviceWorkload(w)
    s = _shape(L, layer, w)
    b = layer.LayerBuffers(s, "cuda", fused_gather=fused)
    layer.forward(dw.x, dw.w_router, dw.bias, dw.w_gu, dw.w_down, s, b)
    torch.cuda.synchronize()
    ref = _oracle(w)
    np.testing.assert_array_equal(b.topk_idx.cpu().numpy(), ref["topk_idx"])
    np.testing.assert_array_equal(b.offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(b.row_of.cpu().numpy(), ref["row_of"])
    np.testing.assert_array_equal(b.src_token.cpu().numpy(), ref["src_token"])
    assert_close(host(b.H), ref["H"], w.dtype, "H")
    assert_close(host(b.Y), ref["Y"], w.dtype, "Y")
    mx, mean = assert_close(host(b.out), ref["out"], w.dtype, "out")
    print(f"{name} fused={fused}: out max rel {mx:.2e} mean rel {mean:.2e}")


def test_layer_graph_replay_with_new_routing(LY):
    """Captured once, replayed on new inputs: group sizes change on the device only."""
    L, layer = LY
    w = mi.WORKLOADS["small_sigmoid"]
    dw = DeviceWorkload(w)
    s = _shape(L, layer, w)
    b = layer.LayerBuffers(s, "cuda")
    x_static = dw.x.clone()
    xs = [dw.x.clone()]
    for seed in (101, 202):
        xi = torch.empty_like(dw.x)
        mi.randn_torch(seed, mi.X, 0, w.T, w.d, 1.0, w.dtype, "cuda", out=xi)
        xs.append(xi)
    eager = []
    for xi in xs:
        layer.forward(xi, dw.w_router, dw.bias, dw.w_gu, dw.w_down, s, b)
        eager.append((b.out.clone(), b.offsets.clone()))
    torch.cuda.synchronize()
    assert not torch.equal(eager[0][1], eager[1][1])          # the routings really differ
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        layer.forward(x_static, dw.w_router, dw.bias, dw.w_gu, dw.w_down, s, b)   # warm-up off the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            layer.forward(x_static, dw.w_router, dw.bias, dw.w_gu, dw.w_down, s, b)
    torch.cuda.synchronize()
    for rep in range(2):
        for xi, (want, want_off) in zip(xs, eager):
            x_static.copy_(xi)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(bits(b.offsets), bits(want_off))
            np.testing.assert_array_equal(bits(b.out), bits(want))


def test_layer_deterministic(LY):
    L, layer = LY
    w = mi.WORKLOADS["small_softmax"]
    dw = DeviceWorkload(w)
    s = _shape(L, layer, w)
    outs = []
    for _ in range(2):
        b = layer.LayerBuffers(s, "cuda")
        layer.forward(dw.x, dw.w_router, dw.bias, dw.w_gu, dw.w_down, s, b)
        torch.cuda.synchronize()
        outs.append((bits(b.out), bits(b.H), b.src_token.cpu().numpy()))
    for a, c in zip(*outs):
        np.testing.assert_array_equal(a, c)
