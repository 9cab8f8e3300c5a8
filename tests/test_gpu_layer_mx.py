"""The MXFP8 training step (forward + backward of the router, the experts, the permutation
and the combine) on the GPU vs the MX-mirroring oracle, on the GPU's own routing so the expert path
is compared on identical groups (routing parity is covered by the route tests). dY is one
rounding of an exact product and must match bit for bit. Every other stage is checked
against the oracle's functions applied to the GPU's own inputs of that stage (bf16
tolerance: one rounding apart), and the whole step against the independent MX oracle with
the end-to-end MXFP8 gate. A forced routing with an empty group checks that its weight
gradients come back as zeros."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as O
from tests.gpu_util import DeviceWorkload, assert_close, assert_close_mx_e2e, bits, host, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def LY():
    from dropless_mixture_experts_device_amd import _lib, layer
    return _lib, layer


def _step(L, layer, w, topk=None, fused=True):
    dw = DeviceWorkload(w)
    s = layer.LayerShape(T=w.T, d=w.d, f=w.f, E=w.E, k=w.k, shared=bool(w.shared_f),
                         score=L.MOE_SOFTMAX if w.score == "softmax" else L.MOE_SIGMOID)
    mw = layer.MxWeights(s, "cuda")
    mw.quantise(dw.w_gu, dw.w_down)
    b = layer.MxBuffers(s, "cuda")
    if topk is not None:
        b.topk_idx.copy_(torch.from_numpy(topk[0]).cuda())
        b.topk_w.copy_(torch.from_numpy(topk[1]).cuda())
    layer.forward_mx(dw.x, dw.w_router, dw.bias, mw, s, b, routed=topk is not None)
    d_out = mi.randn_torch(w.seed, mi.D_OUT, 0, w.T, w.d, 1.0, "bf16", "cuda")
    layer.backward_mx(dw.x, d_out, mw, s, b, w_router=dw.w_router if topk is None else None,
                      fuse_swiglu_quant=fused, fuse_combine_quant=fused)
    if fused:
        # the stage checks read dY, dH and dGU: the standalone kernels write the exact values
        # the fused epilogue and quantisers formed (equal bytes, checked in the fused tests)
        q_dnT, s_dnT = mw.dn_T()
        L.moe_grouped_gemm(b.q_dy, q_dnT, b.dH, b.offsets, L.MOE_EPI_NONE, workspace=b.ws_gemm1, a_scale=b.s_dy,
                           b_scale=s_dnT)
        tk = w.T * w.k
        L.moe_combine_backward(d_out, b.topk_w, b.row_of, b.dY[:tk], dy_shared=b.dY[tk:] if s.shared else None)
        L.moe_swiglu_backward(b.dH, b.GU, b.dGU)
    torch.cuda.synchronize()
    return b


def _oracle(w, b, routed_here=True):
    idx = b.topk_idx.cpu().numpy()
    wt = b.topk_w.cpu().numpy().astype(np.float64)
    gu = lambda e: mi.w_gate_up_np(w, e)
    dn = lambda e: mi.w_down_np(w, e)
    fwd = O.layer_forward(mi.x_np(w), mi.w_router_np(w), mi.expert_bias(w), w.k, w.score, gu, dn, w.E,
                          shared=bool(w.shared_f), rnd=O.round_bf16, topk=(idx, wt), mx=True)
    d_out = mi.randn_np(w.seed, mi.D_OUT, 0, w.T, w.d, 1.0, "bf16").astype(np.float64)
    if routed_here:
        # the forward's keys (the GPU's selection is the oracle's, checked by the route tests)
        fwd["keys"] = O.router_keys(mi.x_np(w), mi.w_router_np(w), mi.expert_bias(w))
    router = (mi.x_np(w), mi.w_router_np(w), w.score) if routed_here else None
    bwd = O.layer_backward(fwd, d_out, gu, dn, w.E, shared=bool(w.shared_f), rnd=O.round_bf16, mx=True,
                           router=router)
    return fwd, bwd


def _stage_refs(w, b, x, d_out, router):
    """Each stage of the step recomputed by the oracle's functions from the GPU's own inputs
    to that stage, so a mismatch points at one kernel."""
    f64 = lambda t: host(t)
    off = b.offsets.cpu().numpy().astype(np.int64)
    src = b.src_token.cpu().numpy()
    ro = b.row_of.cpu().numpy()
    wt = b.topk_w.cpu().numpy().astype(np.float64)
    H, GU, Y, dY, dH, dGU, dXp = (f64(t) for t in (b.H, b.GU, b.Y, b.dY, b.dH, b.dGU, b.dXp))
    tk, f = w.T * w.k, w.f
    xq, Hq, dYq, dGUq = O.mx_q_rows(x), O.mx_q_rows(H), O.mx_q_rows(dY), O.mx_q_rows(dGU)
    ref = {n: np.zeros_like(a) for n, a in (("H", H), ("GU", GU), ("Y", Y), ("dH", dH), ("dX_perm", dXp))}
    ref["dW_gu"] = {}
    ref["dW_down"] = {}
    for g in range(len(off) - 1):
        lo, hi = off[g], off[g + 1]
        if hi == lo:
            continue
        Wgu, Wd = mi.w_gate_up_np(w, g).astype(np.float64), mi.w_down_np(w, g).astype(np.float64)
        Gm, Um = O.expert_gate_up(xq[src[lo:hi]], O.mx_q_rows(Wgu))
        ref["GU"][lo:hi] = O.round_bf16(np.concatenate([Gm, Um], 1))
        ref["H"][lo:hi] = O.round_bf16(O.silu(Gm) * Um)
        ref["Y"][lo:hi] = O.round_bf16(Hq[lo:hi] @ O.mx_q_rows(Wd).T)
        ref["dH"][lo:hi] = O.round_bf16(dYq[lo:hi] @ O.mx_q_rows(Wd.T).T)
        ref["dX_perm"][lo:hi] = O.round_bf16(dGUq[lo:hi] @ O.mx_q_rows(Wgu.T).T)
        one = np.array([0, hi - lo])
        col = lambda a: O.mx_quantize_colwise_grouped(a, one)[2]
        ref["dW_down"][g] = O.round_bf16(col(dY[lo:hi]).T @ col(H[lo:hi]))
        ref["dW_gu"][g] = O.round_bf16(col(dGU[lo:hi]).T @ col(x[src[lo:hi]]))
    Gs, Us = GU[:, :f], GU[:, f:]
    ref["dGU"] = np.concatenate([O.round_bf16(dH * Us * O.silu_grad(Gs)), O.round_bf16(dH * O.silu(Gs))], 1)
    shared = len(off) - 1 > w.E
    ref["out"] = O.combine(Y[:tk], wt, ro, Y[tk:] if shared else None, O.round_bf16)
    ref["dY"], ref["dw"] = O.combine_backward(d_out, Y[:tk], wt, ro, O.round_bf16)
    ref["dx"] = O.permute_backward(dXp[:tk], ro, dXp[tk:] if shared else None, O.round_bf16)
    if router:
        # the router's backward from the GPU's keys, selection and routing-weight gradient
        dk = O.topk_weights_backward(host(b.keys), b.topk_idx.cpu().numpy(), host(b.dw), w.score)
        ref["dW_router"], dx_r, ref["d_bias"] = O.router_backward(x, mi.w_router_np(w), dk)
        ref["dx"] = O.round_bf16(ref["dx"] + dx_r)
    return ref


def _compare(w, b, fwd, bwd, router=True):
    tk = w.T * w.k
    np.testing.assert_array_equal(b.offsets.cpu().numpy(), fwd["offsets"])
    np.testing.assert_array_equal(b.row_of.cpu().numpy(), fwd["row_of"])
    np.testing.assert_array_equal(b.src_token.cpu().numpy(), fwd["src_token"])
    counts = np.diff(fwd["offsets"])
    live = np.flatnonzero(counts)
    x = mi.x_np(w).astype(np.float64)
    d_out = mi.randn_np(w.seed, mi.D_OUT, 0, w.T, w.d, 1.0, "bf16").astype(np.float64)
    # stage by stage, each kernel on the GPU's own inputs
    st = _stage_refs(w, b, x, d_out, router)
    got = {"H": host(b.H), "GU": host(b.GU), "Y": host(b.Y), "out": host(b.out), "dH": host(b.dH),
           "dGU": host(b.dGU), "dX_perm": host(b.dXp), "dx": host(b.dx)}
    dWgu, dWd = host(b.dW_gu), host(b.dW_down)
    np.testing.assert_array_equal(host(b.dY[:tk]), st["dY"])            # w * d_out, one rounding
    assert_close(host(b.dw), st["dw"], "f32", "dw (stage)")
    worst = 0.0
    for n, a in got.items():
        worst = max(worst, assert_close(a, st[n], "bf16", f"{n} (stage)")[0])
    for g in range(len(counts)):
        if counts[g] == 0:
            assert np.all(dWgu[g] == 0) and np.all(dWd[g] == 0), f"empty group {g}: weight gradients must be zero"
            continue
        worst = max(worst, assert_close(dWgu[g], st["dW_gu"][g], "bf16", f"dW_gu[{g}] (stage)")[0])
        worst = max(worst, assert_close(dWd[g], st["dW_down"][g], "bf16", f"dW_down[{g}] (stage)")[0])
    if router:
        assert_close(host(b.dW_router), st["dW_router"], "f32", "dW_router (stage)")
        assert_close(host(b.d_bias), st["d_bias"], "f32", "d_bias (stage)")
    # end to end against the independent MX oracle
    e2e = {"H": (got["H"], fwd["H"]), "Y": (got["Y"], fwd["Y"]), "out": (got["out"], fwd["out"]),
           "dw": (host(b.dw), bwd["dw"]), "dX_perm": (got["dX_perm"], bwd["dX_perm"]), "dx": (got["dx"], bwd["dx"]),
           "dW_gu": (dWgu[live], np.stack([bwd["dW_gu"][g] for g in live])),
           "dW_down": (dWd[live], np.stack([bwd["dW_down"][g] for g in live]))}
    if router:
        e2e["dW_router"] = (host(b.dW_router), bwd["dW_router"])
        e2e["d_bias"] = (host(b.d_bias), bwd["d_bias"])
    msg = []
    for n, (a, r) in e2e.items():
        mx, mean, q = assert_close_mx_e2e(a, r, f"{n} (end to end)")
        msg.append(f"{n} {mx:.1e}/{q:.1e}/{mean:.1e}")
    print(f"stage-wise worst max rel {worst:.2e}; end to end (max/q99.99/mean) " + " ".join(msg))


def test_mx_step_small(LY):
    L, layer = LY
    w = mi.WORKLOADS["small_mxfp8"]
    b = _step(L, layer, w)
    fwd, bwd = _oracle(w, b)
    _compare(w, b, fwd, bwd)
    # the two-kernel SwiGLU backward + quantisation gives the same step, byte for byte
    u = _step(L, layer, w, fused=False)
    for n in ("q_dy", "s_dy", "dY", "q_dgu", "s_dgu", "dGU", "dH", "dXp", "dW_gu", "dW_down", "dx", "dw", "dW_router",
              "d_bias"):
        np.testing.assert_array_equal(bits(getattr(b, n)), bits(getattr(u, n)), err_msg=n)
    # column-wise copies: the group-major blocks written (capacity past block_start[G] is unused)
    nb = int(b.bs[-1].item())
    assert nb == int(u.bs[-1].item())
    cols = 2 * w.f
    for n, per in (("qc_dgu", 32 * cols), ("sc_dgu", cols), ("qc_dy", 32 * w.d), ("sc_dy", w.d)):
        np.testing.assert_array_equal(getattr(b, n).reshape(-1)[:per * nb].cpu().numpy(),
                                      getattr(u, n).reshape(-1)[:per * nb].cpu().numpy(), err_msg=n)


def test_mx_step_mid_end_to_end(LY):
    """The MXFP8 step with every forward and data-gradient contraction 1024 long (T=1024,
    d=f=1024, 8 experts + shared, k=2), stage by stage and end to end against the independent
    MX oracle; the forward output, the input gradient and the router's gradients also hold the
    6e-2 bound on every element."""
    L, layer = LY
    w = mi.WORKLOADS["mid_mxfp8"]
    b = _step(L, layer, w)
    fwd, bwd = _oracle(w, b)
    _compare(w, b, fwd, bwd)
    for n, got, ref in (("out", host(b.out), fwd["out"]), ("dx", host(b.dx), bwd["dx"]),
                        ("dW_router", host(b.dW_router), bwd["dW_router"]), ("d_bias", host(b.d_bias), bwd["d_bias"])):
        mx, mean = rel_err(got, ref)
        assert mx <= 6e-2, f"{n} (end to end, every element): max {mx:.3e}"
        assert got.size < 1024 or mean <= 2e-3, f"{n} (end to end): mean {mean:.3e}"


def test_mx_step_forced_routing_with_empty_group(LY):
    """Experts 0..3 of 12 take every token (expert 5 and others stay empty)."""
    L, layer = LY
    w = mi.WORKLOADS["small_mxfp8"]
    g = np.random.Generator(np.random.PCG64(8))
    idx = np.stack([g.permutation(4)[:w.k] for _ in range(w.T)]).astype(np.int32)
    wt = g.random((w.T, w.k)).astype(np.float32)
    wt /= wt.sum(1, keepdims=True)
    b = _step(L, layer, w, topk=(idx, wt))
    fwd, bwd = _oracle(w, b, routed_here=False)
    assert np.diff(fwd["offsets"])[5] == 0
    _compare(w, b, fwd, bwd, router=False)


def test_mx_step_dsv3_sampled(LY):
    """The full DeepSeek-V3-shaped MXFP8 step (T=8192, d=7168, f=2048, 256 experts + shared,
    k=8) in the configuration the benchmark times, checked stage by stage on sampled rows of
    a large, a small and the shared group, whole weight gradients of the smallest group and
    sampled gradient rows of the largest, sampled tokens of out, dw and dx, and the whole
    router-weight and bias gradients."""
    L, layer = LY
    w = mi.WORKLOADS["dsv3_mxfp8"]
    b = _step(L, layer, w)
    off = b.offsets.cpu().numpy().astype(np.int64)
    src = b.src_token.cpu().numpy()
    counts = np.diff(off)
    tk, f, d = w.T * w.k, w.f, w.d
    rng = np.random.Generator(np.random.PCG64(17))
    big, small = int(np.argmax(counts[:w.E])), int(np.argmin(counts[:w.E]))
    groups = [big, small, w.E]
    rows = {g: np.unique(np.concatenate([[off[g], off[g + 1] - 1], rng.integers(off[g], off[g + 1], 4)]))
            for g in groups}
    pick = lambda t, r: host(t[torch.from_numpy(np.asarray(r)).cuda()])
    for g in groups:
        r = rows[g]
        Wgu, Wd = mi.w_gate_up_np(w, g).astype(np.float64), mi.w_down_np(w, g).astype(np.float64)
        xr = mi.randn_np(w.seed, mi.X, 0, src[r], d, w.sigma_x, "bf16").astype(np.float64)
        Gm, Um = O.expert_gate_up(O.mx_q_rows(xr), O.mx_q_rows(Wgu))
        assert_close(pick(b.GU, r), O.round_bf16(np.concatenate([Gm, Um], 1)), "bf16", f"GU group {g}")
        assert_close(pick(b.H, r), O.round_bf16(O.silu(Gm) * Um), "bf16", f"H group {g}")
        assert_close(pick(b.Y, r), O.round_bf16(O.mx_q_rows(pick(b.H, r)) @ O.mx_q_rows(Wd).T), "bf16",
                     f"Y group {g}")
        assert_close(pick(b.dH, r), O.round_bf16(O.mx_q_rows(pick(b.dY, r)) @ O.mx_q_rows(Wd.T).T), "bf16",
                     f"dH group {g}")
        assert_close(pick(b.dXp, r), O.round_bf16(O.mx_q_rows(pick(b.dGU, r)) @ O.mx_q_rows(Wgu.T).T), "bf16",
                     f"dX_perm group {g}")
    # weight gradients: all of the smallest group, sampled output rows of the largest
    for g, sel_d, sel_f in ((small, np.arange(d), np.arange(2 * f)),
                            (big, rng.integers(0, d, 16), rng.integers(0, 2 * f, 16))):
        lo, hi = off[g], off[g + 1]
        one = np.array([0, hi - lo])
        col = lambda a: O.mx_quantize_colwise_grouped(a, one)[2]
        dY_g, H_g, dGU_g = host(b.dY[lo:hi]), host(b.H[lo:hi]), host(b.dGU[lo:hi])
        x_g = mi.randn_np(w.seed, mi.X, 0, src[lo:hi], d, w.sigma_x, "bf16").astype(np.float64)
        want_dn = O.round_bf16(col(dY_g[:, sel_d]).T @ col(H_g))
        want_gu = O.round_bf16(col(dGU_g[:, sel_f]).T @ col(x_g))
        assert_close(host(b.dW_down[g][torch.from_numpy(sel_d).cuda()]), want_dn, "bf16", f"dW_down[{g}]")
        assert_close(host(b.dW_gu[g][torch.from_numpy(sel_f).cuda()]), want_gu, "bf16", f"dW_gu[{g}]")
    # per-token steps: combine, its transpose and the permutation's transpose on sampled tokens
    toks = np.unique(np.concatenate([[0, w.T - 1], rng.integers(0, w.T, 30)]))
    ro = b.row_of.cpu().numpy()[toks]
    wt = b.topk_w.cpu().numpy()[toks].astype(np.float64)
    need = ro.reshape(-1)
    local = np.arange(need.size).reshape(len(toks), w.k)
    Y_r, dXp_r = pick(b.Y, need), pick(b.dXp, need)
    d_out = mi.randn_np(w.seed, mi.D_OUT, 0, toks, d, 1.0, "bf16").astype(np.float64)
    assert_close(pick(b.out, toks), O.combine(Y_r, wt, local, pick(b.Y, tk + toks), O.round_bf16), "bf16", "out")
    want_dy, want_dw = O.combine_backward(d_out, Y_r, wt, local, O.round_bf16)
    np.testing.assert_array_equal(pick(b.dY, need), want_dy[local.reshape(-1)])
    assert_close(pick(b.dw, toks), want_dw, "f32", "dw")
    # the router's backward from the GPU's keys and dw: its share of dx on the sampled tokens,
    # and the whole router-weight and bias gradients
    dk = O.topk_weights_backward(host(b.keys), b.topk_idx.cpu().numpy(), host(b.dw), w.score)
    wr = mi.w_router_np(w).astype(np.float64)
    dx_exp = O.permute_backward(dXp_r, local, pick(b.dXp, tk + toks), O.round_bf16)
    assert_close(pick(b.dx, toks), O.round_bf16(dx_exp + dk[toks] @ wr), "bf16", "dx")
    dWr, _, db = O.router_backward(mi.x_np(w), wr, dk)
    assert_close(host(b.dW_router), dWr, "f32", "dW_router")
    assert_close(host(b.d_bias), db, "f32", "d_bias")


def test_mx_step_graph_replay_with_new_inputs(LY):
    """The whole MXFP8 training step (weight quantisation, forward, backward with the router
    backward and the fused SwiGLU-backward quantiser) captured once in a HIP graph and
    replayed on new inputs whose routing and group sizes differ: every replay, with eager
    work and synchronisations between replays, equals the eager step bit for bit."""
    L, layer = LY
    w = mi.WORKLOADS["small_mxfp8"]
    dw = DeviceWorkload(w)
    s = layer.LayerShape(T=w.T, d=w.d, f=w.f, E=w.E, k=w.k, shared=bool(w.shared_f),
                         score=L.MOE_SOFTMAX if w.score == "softmax" else L.MOE_SIGMOID)
    mw = layer.MxWeights(s, "cuda")
    b = layer.MxBuffers(s, "cuda")
    x_static = dw.x.clone()
    d_static = mi.randn_torch(w.seed, mi.D_OUT, 0, w.T, w.d, 1.0, "bf16", "cuda")
    inputs = [(dw.x.clone(), d_static.clone())]
    for seed in (301, 302):
        xi, di = torch.empty_like(dw.x), torch.empty_like(d_static)
        mi.randn_torch(seed, mi.X, 0, w.T, w.d, 1.0, w.dtype, "cuda", out=xi)
        mi.randn_torch(seed, mi.D_OUT, 0, w.T, w.d, 1.0, "bf16", "cuda", out=di)
        inputs.append((xi, di))
    names = ("out", "dx", "dW_gu", "dW_down", "dW_router", "d_bias", "offsets")

    def step(x, d_out):
        mw.quantise(dw.w_gu, dw.w_down)
        layer.forward_mx(x, dw.w_router, dw.bias, mw, s, b)
        layer.backward_mx(x, d_out, mw, s, b, w_router=dw.w_router)

    eager = []
    for xi, di in inputs:
        step(xi, di)
        torch.cuda.synchronize()
        eager.append({n: bits(getattr(b, n)).copy() for n in names})
    assert not np.array_equal(eager[0]["offsets"], eager[1]["offsets"])   # the routings really differ
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step(x_static, d_static)                       # warm-up off the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            step(x_static, d_static)
    torch.cuda.synchronize()
    for rep in range(2):
        for (xi, di), want in zip(inputs, eager):
            x_static.copy_(xi)
            d_static.copy_(di)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for n in names:
                np.testing.assert_array_equal(bits(getattr(b, n)), want[n], err_msg=f"{n}, replay {rep}")


@pytest.mark.parametrize("name", ["small_mxfp8", "mid_mxfp8"])
def test_mx_step_fused_h_quant_equals_two_pass(LY, name):
    """The step with its fusions (H quantised in GEMM 1's epilogue, bf16 H not written; the
    SwiGLU backward and dGU's quantisation in dgrad 2's epilogue; dY formed in its quantiser)
    equals, bit for bit, the step with every intermediate written out and quantised by the
    standalone kernels: the quantised copies of H and dGU, the block prefix, Y, the output,
    dX_perm and every gradient."""
    L, layer = LY
    w = mi.WORKLOADS[name]
    dw = DeviceWorkload(w)
    s = layer.LayerShape(T=w.T, d=w.d, f=w.f, E=w.E, k=w.k, shared=bool(w.shared_f),
                         score=L.MOE_SOFTMAX if w.score == "softmax" else L.MOE_SIGMOID)
    mw = layer.MxWeights(s, "cuda")
    mw.quantise(dw.w_gu, dw.w_down)
    d_out = mi.randn_torch(w.seed, mi.D_OUT, 0, w.T, w.d, 1.0, "bf16", "cuda")
    names = ("q_h", "s_h", "qc_h", "sc_h", "bs", "Y", "out", "q_dgu", "s_dgu", "qc_dgu", "sc_dgu", "dXp", "dx",
             "dW_gu", "dW_down", "dW_router", "d_bias")
    got = []
    for fused in (False, True):
        b = layer.MxBuffers(s, "cuda")
        for n in ("qc_h", "sc_h", "qc_dgu", "sc_dgu"):
            getattr(b, n).fill_(0x5A)                    # capacity past the last group: untouched by both
        layer.forward_mx(dw.x, dw.w_router, dw.bias, mw, s, b, fuse_h_quant=fused, write_h=not fused)
        layer.backward_mx(dw.x, d_out, mw, s, b, w_router=dw.w_router, fuse_swiglu_quant=fused,
                          fuse_combine_quant=fused, swiglu_in_dgrad2=fused)
        torch.cuda.synchronize()
        got.append({n: bits(getattr(b, n)).copy() for n in names})
    for n in names:
        np.testing.assert_array_equal(got[1][n], got[0][n], err_msg=n)
