"""moe_route_backward on the GPU vs the oracle. The GPU call takes the oracle's own keys,
selection and permutation as inputs (with seeded x, w_router and routing-weight gradient), so
the comparison is of the backward alone: the keys' gradient, the router-weight and bias
gradients (fp32 sums) and the router's share of the input gradient (one rounding to the
storage dtype) against topk_weights_backward and router_backward."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, dev, dev_i32, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    from dropless_mixture_experts_device_amd import _lib
    return _lib


def _problem(T, d, E, k, score, dtype, seed, bias_skew=0.0):
    x = mi.randn_np(seed, mi.X, 0, T, d, 1.0, dtype)
    w = mi.randn_np(seed, mi.W_ROUTER, 0, E, d, 0.05, dtype)
    b = (bias_skew * (np.arange(E) / max(E - 1, 1) - 0.5)).astype(np.float32)
    keys = O.router_keys(x, w, b)
    idx = O.select_topk(keys, k)
    g = mi.randn_np(seed, mi.D_TOPK_W, 0, T, k, 1.0, "f32")
    return x, w, keys, idx, g


def _run(L, x, w, keys, idx, g, E, score, dtype, outputs=("sel", "dx", "dw", "db")):
    T, d = x.shape
    k = idx.shape[1]
    offsets, row_of, src = O.permutation(idx, E)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {
        "sel": torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda"),
        "dx": torch.full((T, d), float("nan"), dtype=dt, device="cuda"),
        "dw": torch.full((E, d), float("nan"), dtype=torch.float32, device="cuda"),
        "db": torch.full((E,), float("nan"), dtype=torch.float32, device="cuda"),
    }
    out = {n: (t if n in outputs else None) for n, t in out.items()}
    nb = L.moe_workspace_bytes(L.MOE_OP_ROUTE_BWD, T, d, E, k, 0)
    ws = torch.empty((nb,), dtype=torch.uint8, device="cuda")
    sc = L.MOE_SOFTMAX if score == "softmax" else L.MOE_SIGMOID
    L.moe_route_backward(dev(x, dtype), dev(w, dtype), torch.from_numpy(np.ascontiguousarray(keys, np.float32)).cuda(),
                         dev_i32(idx), torch.from_numpy(np.ascontiguousarray(g, np.float32)).cuda(), sc,
                         dev_i32(row_of), offsets=dev_i32(offsets), src_token=dev_i32(src),
                         d_keys_sel=out["sel"], d_x=out["dx"], d_w_router=out["dw"], d_bias=out["db"], workspace=ws)
    torch.cuda.synchronize()
    return {n: (None if t is None else host(t)) for n, t in out.items()}


def _check(got, x, w, keys, idx, g, score, dtype):
    G = O.topk_weights_backward(keys, idx, g, score)
    dW, dx, db = O.router_backward(x, w, G)
    if got["sel"] is not None:
        assert_close(got["sel"], np.take_along_axis(G, idx.astype(np.int64), axis=1), "f32", "d_keys_sel")
    if got["dx"] is not None:
        rnd = O.round_bf16 if dtype == "bf16" else O.round_f32
        assert_close(got["dx"], rnd(dx), dtype, "d_x")
    if got["dw"] is not None:
        assert_close(got["dw"], dW, "f32", "d_w_router")
        unused = np.setdiff1d(np.arange(w.shape[0]), idx)
        assert np.all(got["dw"][unused] == 0.0), "experts no token picked get a zero gradient"
    if got["db"] is not None:
        assert_close(got["db"], db, "f32", "d_bias")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("T,d,E,k", [(1000, 256, 16, 4), (777, 320, 24, 6), (64, 2056, 8, 2), (5, 128, 16, 16),
                                     (33, 64, 128, 1), (20, 7168, 256, 8), (300, 4104, 64, 8),
                                     (3000, 264, 4, 2)])
def test_route_backward(L, dtype, score, T, d, E, k):
    # d = 2056 and 4104 end in a partial column block of the weight gradient; E = 128 and 256
    # with few tokens leave most experts without rows; k = E = 16 selects every expert;
    # T = 3000 over 4 experts gives groups of many 256-row chunks with a ragged last chunk
    x, w, keys, idx, g = _problem(T, d, E, k, score, dtype, seed=T + d + E + k, bias_skew=1.0)
    got = _run(L, x, w, keys, idx, g, E, score, dtype)
    _check(got, x, w, keys, idx, g, score, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_route_backward_accumulates_into_dx(L, dtype):
    """accumulate_dx: the router's share is added to the incoming input gradient, one rounding."""
    T, d, E, k = 300, 1032, 32, 4
    x, w, keys, idx, g = _problem(T, d, E, k, "sigmoid", dtype, seed=9, bias_skew=0.5)
    offsets, row_of, src = O.permutation(idx, E)
    prior = mi.randn_np(9, mi.D_OUT, 0, T, d, 0.02, dtype)
    dx = dev(prior, dtype)
    nb = L.moe_workspace_bytes(L.MOE_OP_ROUTE_BWD, T, d, E, k, 0)
    L.moe_route_backward(dev(x, dtype), dev(w, dtype), dev(keys), dev_i32(idx), dev(g), L.MOE_SIGMOID, dev_i32(row_of), offsets=dev_i32(offsets),
                         src_token=dev_i32(src), d_x=dx, accumulate_dx=True,
                         workspace=torch.empty((nb,), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    _, dx_r, _ = O.router_backward(x, w, O.topk_weights_backward(keys, idx, g, "sigmoid"))
    rnd = O.round_bf16 if dtype == "bf16" else O.round_f32
    assert_close(host(dx), rnd(prior + dx_r), dtype, "d_x accumulated")


@pytest.mark.parametrize("dtype,shared", [("bf16", True), ("bf16", False), ("f32", True)])
def test_route_backward_forms_unpermute(L, dtype, shared):
    """d_x_perm: the dx pass forms the permutation's transpose itself; the bytes equal
    moe_combine without weights followed by the accumulate mode."""
    T, d, E, k = 300, 1032, 32, 6
    x, w, keys, idx, g = _problem(T, d, E, k, "softmax", dtype, seed=13)
    offsets, row_of, src = O.permutation(idx, E, shared_rows=T if shared else 0)
    rows = T * k + (T if shared else 0)
    dxp = dev(mi.randn_np(13, mi.D_OUT, 2, rows, d, 0.05, dtype), dtype)
    nb = L.moe_workspace_bytes(L.MOE_OP_ROUTE_BWD, T, d, E, k, 0)
    common = dict(offsets=dev_i32(offsets), src_token=dev_i32(src),
                  workspace=torch.empty((nb,), dtype=torch.uint8, device="cuda"))
    args = (dev(x, dtype), dev(w, dtype), dev(keys), dev_i32(idx), dev(g), L.MOE_SOFTMAX, dev_i32(row_of))
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    fused = torch.full((T, d), float("nan"), dtype=dt, device="cuda")
    L.moe_route_backward(*args, d_x=fused, d_x_perm=dxp[:T * k], d_x_perm_shared=dxp[T * k:] if shared else None,
                         **common)
    two = torch.full((T, d), float("nan"), dtype=dt, device="cuda")
    L.moe_combine(dxp[:T * k], None, dev_i32(row_of), dxp[T * k:] if shared else None, two)
    L.moe_route_backward(*args, d_x=two, accumulate_dx=True, **common)
    torch.cuda.synchronize()
    from tests.gpu_util import bits
    np.testing.assert_array_equal(bits(fused), bits(two))
    # and against the oracle: the transpose of the permutation (as stored) plus the router's share
    rnd = O.round_bf16 if dtype == "bf16" else O.round_f32
    dxp_h = host(dxp)
    prior = O.permute_backward(dxp_h[:T * k], row_of, dxp_h[T * k:] if shared else None, rnd)
    _, dx_r, _ = O.router_backward(x, w, O.topk_weights_backward(keys, idx, g, "softmax"))
    assert_close(host(fused), rnd(prior + dx_r), dtype, "d_x with the permutation's transpose")


def test_route_backward_outputs_independent(L):
    """Each output may be requested alone; requesting fewer changes none of the others."""
    x, w, keys, idx, g = _problem(500, 512, 32, 4, "sigmoid", "bf16", seed=5)
    full = _run(L, x, w, keys, idx, g, 32, "sigmoid", "bf16")
    for only in (("sel",), ("dx",), ("dw",), ("db",), ("dw", "db")):
        part = _run(L, x, w, keys, idx, g, 32, "sigmoid", "bf16", outputs=only)
        for n in only:
            np.testing.assert_array_equal(part[n], full[n], err_msg=f"{n} alone")


def test_route_backward_deterministic(L):
    x, w, keys, idx, g = _problem(2000, 1024, 64, 8, "softmax", "bf16", seed=6)
    a = _run(L, x, w, keys, idx, g, 64, "softmax", "bf16")
    b = _run(L, x, w, keys, idx, g, 64, "softmax", "bf16")
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)


def test_route_backward_no_tokens(L):
    """T = 0: the weight and bias gradients are zero and nothing else is touched."""
    E, d = 12, 256
    dw = torch.full((E, d), float("nan"), dtype=torch.float32, device="cuda")
    db = torch.full((E,), float("nan"), dtype=torch.float32, device="cuda")
    x = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((E, d), dtype=torch.bfloat16, device="cuda")
    e = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    ws = torch.empty((L.moe_workspace_bytes(L.MOE_OP_ROUTE_BWD, 0, d, E, 2, 0),), dtype=torch.uint8, device="cuda")
    L.moe_route_backward(x, wr, torch.empty((0, E), device="cuda"), e, torch.empty((0, 2), device="cuda"),
                         L.MOE_SIGMOID, e, offsets=torch.zeros(E + 1, dtype=torch.int32, device="cuda"),
                         src_token=torch.empty(0, dtype=torch.int32, device="cuda"), d_w_router=dw, d_bias=db,
                         workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(dw == 0).item() and torch.all(db == 0).item()


def test_route_backward_dsv3_full(L):
    """DeepSeek-V3 router shapes (T = 8192, d = 7168, 256 experts, top-8 sigmoid, Zipf bias)
    in the launch configuration of the training step, every output against the oracle."""
    w = mi.WORKLOADS["dsv3"]
    x = mi.x_np(w)
    wr = mi.w_router_np(w)
    keys = O.router_keys(x, wr, mi.expert_bias(w))
    idx = O.select_topk(keys, w.k)
    g = mi.randn_np(w.seed, mi.D_TOPK_W, 0, w.T, w.k, 1.0, "f32")
    got = _run(L, x, wr, keys, idx, g, w.E, w.score, w.dtype)
    _check(got, x, wr, keys, idx, g, w.score, w.dtype)
