"""MXFP4 on the GPU vs the oracle: the row-wise quantiser (packed E2M1 codes and E8M0 scale
bytes, bit for bit), the MXFP4 grouped GEMM and the MXFP4 layer forward.

On-grid GEMM inputs (every E2M1 code, scale bytes 126..128) keep every product and partial
sum exact in fp32 at these K, so the GPU result must equal the oracle's fp64 product of the
dequantised operands bit for bit: this pins the E2M1 operand packing, the two-dword scale
selection and the 256-value K slices. Random bf16 inputs quantised by the oracle check the
plain and SwiGLU epilogues against the bf16 gate. The layer forward is checked stage by
stage on the GPU's own inputs of each stage, and as a whole against the independent oracle."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as O
from tests.gpu_util import DeviceWorkload, assert_close, dev, dev_i32, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def LY():
    from dropless_mixture_experts_device_amd import _lib, layer
    return _lib, layer


def pack(codes):
    """One 4-bit code per element -> two per byte, the even element in the low nibble."""
    c = np.asarray(codes, np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def _ws(L, G):
    return torch.empty((L.moe_workspace_bytes(L.MOE_OP_GROUPED_GEMM, 0, 0, 0, 0, G),), dtype=torch.uint8,
                       device="cuda")


# ---- quantiser

def _nasty4(rows, cols, seed, dtype="bf16"):
    """Values exact in `dtype` with a different power-of-two range per row, plus special
    blocks: all zero, signed zeros, a saturating block, a constant power of two, a block small
    enough that its scale byte clamps to 0, and (fp32) subnormal inputs."""
    a = mi.randn_np(seed, mi.X, 0, rows, cols, 1.0, dtype).astype(np.float64)
    g = np.random.Generator(np.random.PCG64(seed))
    a *= np.ldexp(1.0, g.integers(-20, 21, rows))[:, None]
    if rows >= 6 and cols >= 64:
        a[0, :32] = 0.0
        a[1, :32] = -0.0
        a[2, :32] = np.clip(a[2, :32], -4.0, 4.0)
        a[2, 7] = 7.0                                   # scale 2^0: 7 saturates to 6, 6.5 too
        a[2, 8] = -6.5
        a[3, 32:64] = 2.0 ** -7
        a[4, :32] = np.ldexp(np.sign(a[4, :32]) + (a[4, :32] == 0), -126)   # floor(log2 amax) - 2 < -127
        if dtype == "f32":
            a[5, 32:64] = np.ldexp(np.round(a[5, 32:64] / np.max(np.abs(a[5, 32:64])) * 64), -140)
    return a


def _quant4(L, a, dtype="bf16", row_index=None, in_rows=None):
    x = dev(a, dtype)
    rows = a.shape[0] if row_index is None else len(row_index)
    cols = a.shape[1]
    q = torch.full((rows, cols // 2), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((rows, cols // 32), 0xAB, dtype=torch.uint8, device="cuda")
    L.moe_group_quant_mxfp4(x, q, s, row_index=None if row_index is None else dev_i32(row_index))
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("rows,cols,dtype", [(64, 256, "bf16"), (300, 7168, "bf16"), (7, 32, "bf16"),
                                             (50, 96, "f32"), (9, 2048, "f32")])
def test_quant4_rowwise_bit_exact(LY, rows, cols, dtype):
    L, _ = LY
    a = _nasty4(rows, cols, rows + cols, dtype)
    q, s = _quant4(L, a, dtype)
    wq, ws, _ = O.mx4_quantize_rowwise(a)
    np.testing.assert_array_equal(s, ws)
    np.testing.assert_array_equal(q, pack(wq))


def _rounding_sweep4():
    """Blocks whose largest magnitude is 6 or 7 (scale byte 127: the values are rounded as
    they are), the other elements sweeping every E2M1 decision: the grid values, the
    midpoints between neighbours (ties to the even mantissa) and the bf16 values one ulp
    either side of each, values past 6 (saturation), in both signs. All exact in bf16."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = list(grid)
    for m in mids:
        ulp = 2.0 ** (np.frexp(m)[1] - 8)
        vals += [m - ulp, m, m + ulp]
    vals += [6.25, 6.5, 7.0, 0.125, 2.0 ** -20]
    vals = np.array(vals + [-v for v in vals])
    n_rows = -(-len(vals) // 31)
    a = np.zeros((n_rows, 32))
    a[:, 0] = np.where(np.arange(n_rows) % 2 == 0, 6.0, 7.0)
    flat = a[:, 1:].reshape(-1)
    flat[:len(vals)] = vals
    a[:, 1:] = flat.reshape(n_rows, 31)
    return a


def test_quant4_rounding_sweep_bit_exact(LY):
    L, _ = LY
    a = _rounding_sweep4()
    assert np.array_equal(O.round_bf16(a), a)
    q, s = _quant4(L, a)
    wq, ws, _ = O.mx4_quantize_rowwise(a)
    assert np.all(ws == 127)
    np.testing.assert_array_equal(s, ws)
    np.testing.assert_array_equal(q, pack(wq))


def test_quant4_gather_rows_bit_exact(LY):
    """Logical row r reads input row row_index[r] (repeats, any order, out-of-range entries
    clamped into the input)."""
    L, _ = LY
    a = _nasty4(40, 512, 3)
    idx = np.random.Generator(np.random.PCG64(4)).integers(0, 40, 97).astype(np.int64)
    idx[:3] = [-5, 40, 1000]
    q, s = _quant4(L, a, row_index=idx)
    wq, ws, _ = O.mx4_quantize_rowwise(a[np.clip(idx, 0, 39)])
    np.testing.assert_array_equal(s, ws)
    np.testing.assert_array_equal(q, pack(wq))


# ---- grouped GEMM

def _grid_operand4(shape, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    codes = g.integers(0, 16, size=shape).astype(np.uint8)          # every E2M1 code, -0 included
    scales = g.integers(126, 129, size=shape[:-1] + (shape[-1] // 32,)).astype(np.uint8)
    return codes, scales


def _dequant4(codes, scales):
    return O.e2m1_decode(codes) * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)


def _run4(L, A, As, B, Bs, off, M, N, epi, c_dtype, a_rows=None):
    """A and B are one code per element here; they are packed for the GPU."""
    C = torch.full((M, N), float("nan"), dtype=c_dtype, device="cuda")
    L.moe_grouped_gemm(_u8(pack(A)), _u8(pack(B)), C, dev_i32(off), epi,
                       a_rows=None if a_rows is None else dev_i32(a_rows), workspace=_ws(L, B.shape[0]),
                       a_scale=_u8(As), b_scale=_u8(Bs), fp4=True)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("sizes,N,K", [([0, 1, 17, 33, 65, 129, 300, 2], 256, 512), ([700], 192, 256),
                                       ([5, 0, 90], 520, 2048)])
@pytest.mark.parametrize("gather", [False, True])
def test_mx4_gemm_on_grid_bit_exact(LY, sizes, N, K, gather):
    L, _ = LY
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, G = int(off[-1]) + 2, len(sizes)
    A, As = _grid_operand4((M + 5, K), N + K)
    B, Bs = _grid_operand4((G, N, K), G + K)
    a_rows = np.random.Generator(np.random.PCG64(2)).integers(0, M + 5, M).astype(np.int32) if gather else None
    C = host(_run4(L, A, As, B, Bs, off, M, N, L.MOE_EPI_NONE, torch.float32, a_rows))
    want = O.grouped_gemm(_dequant4(A, As), _dequant4(B, Bs), off, a_row_index=a_rows)
    np.testing.assert_array_equal(C[:off[-1]], want)
    assert np.all(np.isnan(C[off[-1]:]))


def test_mx4_gemm_on_grid_bf16_output_is_one_rounding(LY):
    L, _ = LY
    sizes = [33, 0, 260, 1]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, G, N, K = int(off[-1]), len(sizes), 384, 1024
    A, As = _grid_operand4((M, K), 5)
    B, Bs = _grid_operand4((G, N, K), 6)
    C = host(_run4(L, A, As, B, Bs, off, M, N, L.MOE_EPI_NONE, torch.bfloat16))
    want = O.grouped_gemm(_dequant4(A, As), _dequant4(B, Bs), off, rnd=O.round_bf16)
    np.testing.assert_array_equal(C, want)


@pytest.mark.parametrize("epi", ["none", "swiglu"])
def test_mx4_gemm_quantised_random_within_tolerance(LY, epi):
    L, _ = LY
    sizes = [40, 0, 1, 200, 7, 129, 513]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, G, N, K = int(off[-1]), len(sizes), 384, 1024
    nb = 2 * N if epi == "swiglu" else N
    x = mi.randn_np(7, mi.X, 0, M, K, 1.0, "bf16").astype(np.float64)
    W = np.stack([mi.randn_np(7, mi.W_GATE, g, nb, K, 0.02, "bf16") for g in range(G)]).astype(np.float64)
    A, As, Aq = O.mx4_quantize_rowwise(x)
    parts = [O.mx4_quantize_rowwise(W[g]) for g in range(G)]
    B = np.stack([p[0] for p in parts])
    Bs = np.stack([p[1] for p in parts])
    Wq = np.stack([p[2] for p in parts])
    if epi == "none":
        C = _run4(L, A, As, B, Bs, off, M, N, L.MOE_EPI_NONE, torch.bfloat16)
        want = O.grouped_gemm(Aq, Wq, off, rnd=O.round_bf16)
    else:
        C = _run4(L, A, As, B, Bs, off, M, N, L.MOE_EPI_SWIGLU, torch.bfloat16)
        want = O.grouped_swiglu(Aq, Wq, off, rnd=O.round_bf16)
    assert_close(host(C), want, "bf16", f"mx4 {epi}")


# ---- layer forward

def _forward4(L, layer, w):
    dw = DeviceWorkload(w)
    s = layer.LayerShape(T=w.T, d=w.d, f=w.f, E=w.E, k=w.k, shared=bool(w.shared_f),
                         score=L.MOE_SOFTMAX if w.score == "softmax" else L.MOE_SIGMOID)
    mw = layer.Mx4Weights(s, "cuda")
    mw.quantise(dw.w_gu, dw.w_down)
    b = layer.Mx4Buffers(s, "cuda")
    layer.forward_mx4(dw.x, dw.w_router, dw.bias, mw, s, b)
    torch.cuda.synchronize()
    return dw, mw, b


def test_mx4_layer_forward_small(LY):
    """Stage by stage on the GPU's own routing: the quantised weights and x bit for bit, H,
    Y and out within the bf16 gate of the oracle's step applied to the GPU's own input of
    that stage, the quantised H bit for bit; then the whole forward against the independent
    oracle (which mirrors every quantisation) within the bf16 gate on the mean and 6e-2 on
    the 99.99th percentile (a bf16 H one ulp from the oracle's can flip an E2M1 code)."""
    L, layer = LY
    w = mi.WORKLOADS["small_mxfp4"]
    dw, mw, b = _forward4(L, layer, w)
    idx = b.topk_idx.cpu().numpy()
    wt = b.topk_w.cpu().numpy().astype(np.float64)
    gu = lambda e: mi.w_gate_up_np(w, e)
    dn = lambda e: mi.w_down_np(w, e)
    fwd = O.layer_forward(mi.x_np(w), None, None, w.k, w.score, gu, dn, w.E, shared=bool(w.shared_f),
                          rnd=O.round_bf16, topk=(idx, wt), mx4=True)
    np.testing.assert_array_equal(b.offsets.cpu().numpy(), fwd["offsets"])
    np.testing.assert_array_equal(b.row_of.cpu().numpy(), fwd["row_of"])
    np.testing.assert_array_equal(b.src_token.cpu().numpy(), fwd["src_token"])
    x = mi.x_np(w).astype(np.float64)
    xc, xs, xq = O.mx4_quantize_rowwise(x)
    np.testing.assert_array_equal(b.q_x.cpu().numpy(), pack(xc))
    np.testing.assert_array_equal(b.s_x.cpu().numpy(), xs)
    G = w.E + 1
    qgu, sgu, qdn, sdn = (t.cpu().numpy() for t in (mw.q_gu, mw.s_gu, mw.q_dn, mw.s_dn))
    off = fwd["offsets"]
    src = fwd["src_token"]
    H, Y = host(b.H), host(b.Y)
    ref_H, ref_Y = np.zeros_like(H), np.zeros_like(Y)
    hc, hs, hq = O.mx4_quantize_rowwise(H)
    np.testing.assert_array_equal(b.q_h.cpu().numpy(), pack(hc))
    np.testing.assert_array_equal(b.s_h.cpu().numpy(), hs)
    for g in range(G):
        wgc, wgs, wgq = O.mx4_quantize_rowwise(gu(g).astype(np.float64))
        wdc, wds, wdq = O.mx4_quantize_rowwise(dn(g).astype(np.float64))
        np.testing.assert_array_equal(qgu[g], pack(wgc))
        np.testing.assert_array_equal(sgu[g], wgs)
        np.testing.assert_array_equal(qdn[g], pack(wdc))
        np.testing.assert_array_equal(sdn[g], wds)
        lo, hi = int(off[g]), int(off[g + 1])
        if hi == lo:
            continue
        Gm, Um = O.expert_gate_up(xq[src[lo:hi]], wgq)
        ref_H[lo:hi] = O.round_bf16(O.silu(Gm) * Um)
        ref_Y[lo:hi] = O.round_bf16(hq[lo:hi] @ wdq.T)
    assert_close(H, ref_H, "bf16", "H")
    assert_close(Y, ref_Y, "bf16", "Y")
    tk = w.T * w.k
    ro = b.row_of.cpu().numpy()
    assert_close(host(b.out), O.combine(Y[:tk], wt, ro, Y[tk:], O.round_bf16), "bf16", "out")
    # the whole forward against the independent oracle
    for name, got, ref in (("H", H, fwd["H"]), ("Y", Y, fwd["Y"]), ("out", host(b.out), fwd["out"])):
        e = np.sort(np.abs(got - ref).ravel() / np.maximum(np.abs(ref).ravel(), np.sqrt(np.mean(ref * ref))))
        q = float(np.quantile(e, 0.9999))
        print(f"{name}: max {e[-1]:.3e} q99.99 {q:.3e} mean {e.mean():.3e}")
        assert q <= 6e-2 and e.mean() <= 2e-3, (name, q, e.mean())


def test_mx4_layer_forward_dsv3_sampled(LY):
    """The DeepSeek-V3-shaped MXFP4 forward (T=8192, d=7168, f=2048, 256 experts + shared,
    k=8) as the benchmark runs it, checked stage by stage on sampled rows of the largest and
    smallest routed groups and the shared group, and on sampled tokens of out."""
    L, layer = LY
    w = mi.WORKLOADS["dsv3_mxfp4"]
    dw, mw, b = _forward4(L, layer, w)
    off = b.offsets.cpu().numpy().astype(np.int64)
    src = b.src_token.cpu().numpy()
    counts = np.diff(off)
    rng = np.random.Generator(np.random.PCG64(23))
    big, small = int(np.argmax(counts[:w.E])), int(np.argmin(counts[:w.E]))
    pick = lambda t, r: host(t[torch.from_numpy(np.asarray(r)).cuda()])
    for g in (big, small, w.E):
        if counts[g] == 0:
            continue
        r = np.unique(np.concatenate([[off[g], off[g + 1] - 1], rng.integers(off[g], off[g + 1], 4)]))
        Wgu, Wd = mi.w_gate_up_np(w, g).astype(np.float64), mi.w_down_np(w, g).astype(np.float64)
        xr = mi.randn_np(w.seed, mi.X, 0, src[r], w.d, w.sigma_x, "bf16").astype(np.float64)
        Gm, Um = O.expert_gate_up(O.mx4_q_rows(xr), O.mx4_q_rows(Wgu))
        assert_close(pick(b.H, r), O.round_bf16(O.silu(Gm) * Um), "bf16", f"H group {g}")
        hr = pick(b.H, r)
        hc, hs, hq = O.mx4_quantize_rowwise(hr)
        np.testing.assert_array_equal(b.q_h[torch.from_numpy(r).cuda()].cpu().numpy(), pack(hc))
        np.testing.assert_array_equal(b.s_h[torch.from_numpy(r).cuda()].cpu().numpy(), hs)
        assert_close(pick(b.Y, r), O.round_bf16(hq @ O.mx4_q_rows(Wd).T), "bf16", f"Y group {g}")
    toks = np.unique(np.concatenate([[0, w.T - 1], rng.integers(0, w.T, 30)]))
    ro = b.row_of.cpu().numpy()[toks]
    wt = b.topk_w.cpu().numpy()[toks].astype(np.float64)
    need = ro.reshape(-1)
    local = np.arange(need.size).reshape(len(toks), w.k)
    assert_close(pick(b.out, toks), O.combine(pick(b.Y, need), wt, local, pick(b.Y, w.T * w.k + toks),
                                              O.round_bf16), "bf16", "out")


def test_mx4_forward_fused_h_quant_equals_two_pass(LY):
    """H quantised to MXFP4 in GEMM 1's epilogue (bf16 H not written) gives the same codes,
    scales, Y and output, bit for bit, as the bf16 H passed through moe_group_quant_mxfp4."""
    L, layer = LY
    w = mi.WORKLOADS["small_mxfp4"]
    dw = DeviceWorkload(w)
    s = layer.LayerShape(T=w.T, d=w.d, f=w.f, E=w.E, k=w.k, shared=bool(w.shared_f),
                         score=L.MOE_SOFTMAX if w.score == "softmax" else L.MOE_SIGMOID)
    mw = layer.Mx4Weights(s, "cuda")
    mw.quantise(dw.w_gu, dw.w_down)
    got = []
    for fused in (False, True):
        b = layer.Mx4Buffers(s, "cuda")
        layer.forward_mx4(dw.x, dw.w_router, dw.bias, mw, s, b, fuse_h_quant=fused, write_h=not fused)
        torch.cuda.synchronize()
        got.append({n: getattr(b, n).view(torch.uint8).cpu().numpy().copy() for n in ("q_h", "s_h", "Y", "out")})
    for n in got[0]:
        np.testing.assert_array_equal(got[1][n], got[0][n], err_msg=n)
