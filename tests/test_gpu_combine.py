"""moe_combine on the GPU vs the oracle, plus the exact property that combining the gathered
rows with equal weights 1/k restores x bit for bit."""
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


@pytest.mark.parametrize("name,shared", [("tiny", False), ("small_softmax", False), ("small_sigmoid", True),
                                         ("qwen3", False), ("dsv3", True)])
def test_combine_workload(L, name, shared):
    w = mi.WORKLOADS[name]
    x = mi.x_np(w)
    idx, wt, _ = O.route(x, mi.w_router_np(w), mi.expert_bias(w), w.k, w.score)
    _, row_of, _ = O.permutation(idx, w.E)
    rows = w.T * w.k
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    Yd = torch.empty((rows, w.d), dtype=dt, device="cuda")
    mi.randn_torch(w.seed, mi.D_OUT, 5, rows, w.d, 0.5, w.dtype, "cuda", out=Yd)
    Ysd = mi.randn_torch(w.seed, mi.D_OUT, 6, w.T, w.d, 0.5, w.dtype, "cuda") if shared else None
    wt32 = wt.astype(np.float32)                       # the routing weights are stored in fp32
    out = torch.full((w.T, w.d), float("nan"), dtype=dt, device="cuda")
    L.moe_combine(Yd, torch.from_numpy(wt32).cuda(), dev_i32(row_of), Ysd, out)
    torch.cuda.synchronize()
    # the oracle regenerates only the rows the sampled tokens need
    toks = np.arange(w.T) if w.T <= 1024 else np.unique(np.concatenate(
        [[0, w.T - 1], np.random.Generator(np.random.PCG64(1)).integers(0, w.T, 254)]))
    need = row_of[toks].reshape(-1)
    Y_rows = mi.randn_np(w.seed, mi.D_OUT, 5, need, w.d, 0.5, w.dtype)
    local = np.arange(need.size).reshape(len(toks), w.k)
    Ys = mi.randn_np(w.seed, mi.D_OUT, 6, toks, w.d, 0.5, w.dtype) if shared else None
    rnd = O.round_bf16 if w.dtype == "bf16" else O.round_f32
    want = O.combine(Y_rows, wt32[toks], local, Ys, rnd=rnd)
    assert_close(host(out[torch.from_numpy(toks).cuda()]), want, w.dtype, "combine")


@pytest.mark.parametrize("k", [1, 2, 3, 5, 8])   # 3 and 5 take the kernel's runtime-k loop
def test_combine_of_gathered_rows_is_identity(L, k):
    T, E, d = 700, 32, 256
    g = np.random.Generator(np.random.PCG64(k))
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = mi.randn_np(3, mi.X, 0, T, d, 1.0, "bf16")
    _, row_of, src = O.permutation(idx, E)
    xd = dev(x, "bf16")
    out = torch.empty_like(xd)
    L.moe_combine(dev(x[src], "bf16"), torch.full((T, k), 1.0 / k, device="cuda"), dev_i32(row_of), None, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), bits(xd))
