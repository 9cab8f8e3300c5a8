"""The backward's elementwise and data-movement steps on the GPU vs the oracle:
moe_combine_backward (the transpose of the weighted combine, plus the routing weights'
gradient), moe_combine with no weights (the transpose of the permutation's gather) and
moe_swiglu_backward. dY is one rounding of an exact product, so it must match the oracle bit
for bit; sums and transcendental math are held to the storage tolerance."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, bits, dev, dev_i32, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    from dropless_mixture_experts_device_amd import _lib
    return _lib


def _routing(w):
    idx, wt, _ = O.route(mi.x_np(w), mi.w_router_np(w), mi.expert_bias(w), w.k, w.score)
    _, row_of, _ = O.permutation(idx, w.E)
    return wt.astype(np.float32), row_of


@pytest.mark.parametrize("name", ["tiny", "small_softmax", "small_sigmoid"])
def test_combine_backward_full(L, name):
    w = mi.WORKLOADS[name]
    wt32, row_of = _routing(w)
    rows = w.T * w.k
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    d_out = mi.randn_np(w.seed, mi.D_OUT, 0, w.T, w.d, 1.0, w.dtype)
    Y = mi.randn_np(w.seed, mi.D_OUT, 5, rows, w.d, 0.5, w.dtype)
    dy = torch.full((rows, w.d), float("nan"), dtype=dt, device="cuda")
    dys = torch.full((w.T, w.d), float("nan"), dtype=dt, device="cuda")
    dw = torch.full((w.T, w.k), float("nan"), dtype=torch.float32, device="cuda")
    god = dev(d_out, w.dtype)
    L.moe_combine_backward(god, torch.from_numpy(wt32).cuda(), dev_i32(row_of), dy, y=dev(Y, w.dtype),
                           dy_shared=dys, dw=dw)
    torch.cuda.synchronize()
    rnd = O.round_bf16 if w.dtype == "bf16" else O.round_f32
    want_dy, want_dw = O.combine_backward(d_out, Y, wt32, row_of, rnd=rnd)
    np.testing.assert_array_equal(host(dy), want_dy)           # one rounding of an exact product
    np.testing.assert_array_equal(bits(dys), bits(god))         # the shared expert's gradient is d_out
    assert_close(host(dw), want_dw, "f32", "dw")


def test_combine_backward_dsv3_sampled(L):
    """DeepSeek-V3 shapes (T=8192, d=7168, k=8), dy for sampled tokens bit-exact and their dw."""
    w = mi.WORKLOADS["dsv3"]
    wt32, row_of = _routing(w)
    rows = w.T * w.k
    god = mi.randn_torch(w.seed, mi.D_OUT, 0, w.T, w.d, 1.0, "bf16", "cuda")
    Yd = mi.randn_torch(w.seed, mi.D_OUT, 5, rows, w.d, 0.5, "bf16", "cuda")
    dy = torch.empty((rows, w.d), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    L.moe_combine_backward(god, torch.from_numpy(wt32).cuda(), dev_i32(row_of), dy, y=Yd, dw=dw)
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([[0, w.T - 1], np.random.Generator(np.random.PCG64(4)).integers(0, w.T, 60)]))
    need = row_of[toks].reshape(-1)
    d_rows = mi.randn_np(w.seed, mi.D_OUT, 0, toks, w.d, 1.0, "bf16")
    Y_rows = mi.randn_np(w.seed, mi.D_OUT, 5, need, w.d, 0.5, "bf16")
    local = np.arange(need.size).reshape(len(toks), w.k)
    want_dy, want_dw = O.combine_backward(d_rows, Y_rows, wt32[toks], local, rnd=O.round_bf16)
    got_dy = host(dy[torch.from_numpy(need).cuda()])
    np.testing.assert_array_equal(got_dy, want_dy[local.reshape(-1)])
    assert_close(host(dw[torch.from_numpy(toks).cuda()]), want_dw, "f32", "dw")


@pytest.mark.parametrize("shared", [False, True])
def test_unpermute_sum_integer_exact(L, shared):
    """moe_combine without weights is the transpose of the gather: with small-integer rows
    every fp32 partial sum is exact, so it must equal the oracle's permute_backward."""
    T, E, k, d = 900, 24, 6, 192
    g = np.random.Generator(np.random.PCG64(21))
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, row_of, _ = O.permutation(idx, E)
    dXp = mi.integer_valued((T * k, d), -8, 8, 3, 5)
    dXs = mi.integer_valued((T, d), -8, 8, 3, 6) if shared else None
    out = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.moe_combine(dev(dXp, "bf16"), None, dev_i32(row_of), None if dXs is None else dev(dXs, "bf16"), out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), O.permute_backward(dXp, row_of, dXs, rnd=O.round_bf16))


def test_unpermute_sum_random_within_tolerance(L):
    w = mi.WORKLOADS["small_sigmoid"]
    _, row_of = _routing(w)
    rows = w.T * w.k
    dXp = mi.randn_np(w.seed, mi.D_OUT, 7, rows + w.T, w.d, 1.0, "bf16")
    out = torch.empty((w.T, w.d), dtype=torch.bfloat16, device="cuda")
    xd = dev(dXp, "bf16")
    L.moe_combine(xd[:rows], None, dev_i32(row_of), xd[rows:], out)
    torch.cuda.synchronize()
    assert_close(host(out), O.permute_backward(dXp[:rows], row_of, dXp[rows:], rnd=O.round_bf16), "bf16",
                 "unpermute")


@pytest.mark.parametrize("rows,f,dtype", [(300, 384, "bf16"), (77, 64, "f32"), (4096, 2048, "bf16")])
def test_swiglu_backward(L, rows, f, dtype):
    g = mi.randn_np(5, mi.X, 2, rows, f, 2.0, dtype)
    u = mi.randn_np(5, mi.X, 3, rows, f, 1.0, dtype)
    dh = mi.randn_np(5, mi.X, 4, rows, f, 1.0, dtype)
    g[:, :8] = 0.0                                             # silu'(0) = 1/2 and silu(0) = 0 exactly
    gu = np.concatenate([g, u], axis=1)
    dgu = torch.full((rows, 2 * f), float("nan"), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                     device="cuda")
    L.moe_swiglu_backward(dev(dh, dtype), dev(gu, dtype), dgu)
    torch.cuda.synchronize()
    rnd = O.round_bf16 if dtype == "bf16" else O.round_f32
    G, U, dH = g.astype(np.float64), u.astype(np.float64), dh.astype(np.float64)
    want = np.concatenate([rnd(dH * U * O.silu_grad(G)), rnd(dH * O.silu(G))], axis=1)
    got = host(dgu)
    np.testing.assert_array_equal(got[:, :8], want[:, :8])     # g = 0: exact products, one rounding
    np.testing.assert_array_equal(got[:, f:f + 8], 0.0)
    assert_close(got, want, dtype, "swiglu backward")
