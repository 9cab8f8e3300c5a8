"""MXFP8 grouped GEMM on the GPU vs the oracle.

On-grid inputs (E4M3 codes of small integers, per-block scale bytes within +-2 of 127) make
every product and partial sum exact in fp32, so the GPU result must equal the oracle's fp64
product of the dequantised operands bit for bit: this pins the scaled-MFMA operand layout,
the per-lane scale selection and the fp8 tile geometry. Random bf16 inputs quantised by the
oracle's own quantiser then check the plain and SwiGLU epilogues within tolerance."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, bits, dev_i32, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    from dropless_mixture_experts_device_amd import _lib
    return _lib


def _ws(L, G):
    return torch.empty((L.moe_workspace_bytes(L.MOE_OP_GROUPED_GEMM, 0, 0, 0, 0, G),), dtype=torch.uint8,
                       device="cuda")


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def _dequant(codes, scales):
    """value = decode(code) * 2^(scale - 127), blocks of 32 along the last axis."""
    v = O.e4m3_decode(codes)
    s = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)
    return v * s


def _grid_operand(shape, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    vals = g.integers(-2, 3, size=shape).astype(np.float64) * 0.25      # exact E4M3 values
    codes = O.e4m3_encode(O.e4m3_round(vals))
    scales = g.integers(125, 130, size=shape[:-1] + (shape[-1] // 32,)).astype(np.uint8)
    return codes, scales


def _run(L, A, As, B, Bs, off, M, N, epi, c_dtype, a_rows=None):
    C = torch.full((M, N), float("nan"), dtype=c_dtype, device="cuda")
    L.moe_grouped_gemm(_u8(A), _u8(B), C, dev_i32(off), epi, a_rows=None if a_rows is None else dev_i32(a_rows),
                       workspace=_ws(L, B.shape[0]), a_scale=_u8(As), b_scale=_u8(Bs))
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("sizes,N,K", [([0, 1, 17, 33, 65, 129, 300, 2], 256, 512), ([700], 192, 128),
                                       ([5, 0, 90], 520, 2048)])
@pytest.mark.parametrize("gather", [False, True])
def test_mx_gemm_on_grid_bit_exact(L, sizes, N, K, gather):
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, G = int(off[-1]) + 2, len(sizes)
    A, As = _grid_operand((M + 5, K), N + K)
    B, Bs = _grid_operand((G, N, K), G + K)
    a_rows = np.random.Generator(np.random.PCG64(2)).integers(0, M + 5, M).astype(np.int32) if gather else None
    C = host(_run(L, A, As, B, Bs, off, M, N, L.MOE_EPI_NONE, torch.float32, a_rows))
    want = O.grouped_gemm(_dequant(A, As), _dequant(B, Bs), off, a_row_index=a_rows)
    np.testing.assert_array_equal(C[:off[-1]], want)
    assert np.all(np.isnan(C[off[-1]:]))


def test_mx_gemm_on_grid_max_groups(L):
    """The largest block-scaled row-tile launch (1,023 groups: the tile prefix fills the LDS left
    past the operand stages and the two scale-batch slots), with empty, one-row and ragged groups
    and K = 640 (5 MXFP8 stages: a full scale batch, then one clamped to the rows' last dword):
    bit-exact against the oracle; 1,024 groups are refused."""
    G, N, K = 1023, 64, 640
    sizes = np.random.Generator(np.random.PCG64(5)).integers(0, 4, G)
    sizes[::97] = 0
    sizes[5] = 130
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(off[-1])
    A, As = _grid_operand((M, K), 31)
    B, Bs = _grid_operand((G, N, K), 32)
    C = host(_run(L, A, As, B, Bs, off, M, N, L.MOE_EPI_NONE, torch.float32))
    np.testing.assert_array_equal(C, O.grouped_gemm(_dequant(A, As), _dequant(B, Bs), off))
    off2 = np.concatenate([off, [M]]).astype(np.int32)
    B2 = np.concatenate([B, B[:1]])
    Bs2 = np.concatenate([Bs, Bs[:1]])
    with pytest.raises(L.MoeError) as e:
        _run(L, A, As, B2, Bs2, off2, M, N, L.MOE_EPI_NONE, torch.float32)
    assert e.value.status == L.MOE_ENOTSUP


@pytest.mark.parametrize("epi", ["none", "swiglu"])
def test_mx_gemm_quantised_random_within_tolerance(L, epi):
    sizes = [40, 0, 1, 200, 7, 129, 513]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, G, N, K = int(off[-1]), len(sizes), 384, 1024
    nb = 2 * N if epi == "swiglu" else N
    x = mi.randn_np(7, mi.X, 0, M, K, 1.0, "bf16").astype(np.float64)
    W = np.stack([mi.randn_np(7, mi.W_GATE, g, nb, K, 0.02, "bf16") for g in range(G)]).astype(np.float64)
    A, As, Aq = O.mx_quantize_rowwise(x)
    Bq_parts = [O.mx_quantize_rowwise(W[g]) for g in range(G)]
    B = np.stack([p[0] for p in Bq_parts])
    Bs = np.stack([p[1] for p in Bq_parts])
    Wq = np.stack([p[2] for p in Bq_parts])
    if epi == "none":
        C = _run(L, A, As, B, Bs, off, M, N, L.MOE_EPI_NONE, torch.bfloat16)
        want = O.grouped_gemm(Aq, Wq, off, rnd=O.round_bf16)
    else:
        C = _run(L, A, As, B, Bs, off, M, N, L.MOE_EPI_SWIGLU, torch.bfloat16)
        want = O.grouped_swiglu(Aq, Wq, off, rnd=O.round_bf16)
    assert_close(host(C), want, "bf16", f"mx {epi}")


@pytest.mark.parametrize("cdt", ["f32", "bf16"])   # bf16 output takes the K-slice streaming path
def test_mx_gemm_ragged_k_on_grid_bit_exact(L, cdt):
    """Weight-gradient form: C[g] = A_g @ B_g^T over each group's own blocks (multiples of 4
    blocks), the operands in the column-wise quantiser's group-major layout (group g's
    [M, 32 n_g] block at 32*M*offsets[g]), with an empty range whose C[g] must come back as
    zeros, and M, N that leave partial tiles. On-grid operands make every fp32 sum exact, so
    the fp32 output is the exact product and the bf16 output its one nearest-even rounding."""
    blocks = np.array([0, 4, 4, 12, 16, 28], np.int32)          # group K ranges in 32-element blocks
    G, M, N, K = len(blocks) - 1, 192, 320, 32 * int(blocks[-1])
    parts = [(_grid_operand((M, 32 * int(blocks[g + 1] - blocks[g])), 11 + g),
              _grid_operand((N, 32 * int(blocks[g + 1] - blocks[g])), 31 + g)) for g in range(G)]
    flat = lambda arrs, rows, width: np.concatenate([x.reshape(-1) for x in arrs]).reshape(rows, width)
    A = flat([p[0][0] for p in parts], M, K)
    As = flat([p[0][1] for p in parts], M, K // 32)
    B = flat([p[1][0] for p in parts], N, K)
    Bs = flat([p[1][1] for p in parts], N, K // 32)
    C = torch.full((G, M, N), float("nan"), dtype=torch.float32 if cdt == "f32" else torch.bfloat16, device="cuda")
    L.moe_grouped_gemm(_u8(A), _u8(B), C, dev_i32(blocks), L.MOE_EPI_NONE, workspace=_ws(L, G),
                       a_scale=_u8(As), b_scale=_u8(Bs), ragged_k=True)
    torch.cuda.synchronize()
    got = host(C)
    rnd = (lambda v: v) if cdt == "f32" else O.round_bf16
    for g in range(G):
        (Ag, Ags), (Bg, Bgs) = parts[g]
        np.testing.assert_array_equal(got[g], rnd(_dequant(Ag, Ags) @ _dequant(Bg, Bgs).T), err_msg=f"group {g}")


def test_mx_wgrad_quantised_within_tolerance(L):
    """The column-wise quantiser feeding the ragged-K GEMM reproduces the oracle's MXFP8
    weight gradient dW_g = Qcol(dY_g)^T Qcol(H_g) per group, bf16 output."""
    sizes = [37, 0, 1, 160, 128, 300]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows, G, d, f = int(off[-1]), len(sizes), 256, 384
    dY = mi.randn_np(9, mi.D_OUT, 0, rows, d, 1.0, "bf16").astype(np.float64)
    H = mi.randn_np(9, mi.X, 1, rows, f, 0.5, "bf16").astype(np.float64)
    nblk = L.quant_col_blocks(rows, G)
    qa = torch.zeros((d, 32 * nblk), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((d, nblk), dtype=torch.uint8, device="cuda")
    qb = torch.zeros((f, 32 * nblk), dtype=torch.uint8, device="cuda")
    sb = torch.zeros((f, nblk), dtype=torch.uint8, device="cuda")
    bs = torch.empty((G + 1,), dtype=torch.int32, device="cuda")
    offs = dev_i32(off)
    L.moe_group_quant_mxfp8(torch.from_numpy(dY).to(torch.bfloat16).cuda(), qa, sa, axis=1, group_offsets=offs,
                            block_start=bs)
    L.moe_group_quant_mxfp8(torch.from_numpy(H).to(torch.bfloat16).cuda(), qb, sb, axis=1, group_offsets=offs,
                            block_start=bs)
    C = torch.full((G, d, f), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.moe_grouped_gemm(qa, qb, C, bs, L.MOE_EPI_NONE, workspace=_ws(L, G), a_scale=sa, b_scale=sb, ragged_k=True)
    torch.cuda.synchronize()
    got = host(C)
    _, _, dYq = O.mx_quantize_colwise_grouped(dY, off)
    _, _, Hq = O.mx_quantize_colwise_grouped(H, off)
    for g in range(G):
        lo, hi = int(off[g]), int(off[g + 1])
        want = O.round_bf16(dYq[lo:hi].T @ Hq[lo:hi])
        if hi == lo:
            assert np.all(got[g] == 0), "an empty group's weight gradient is written as zeros"
        else:
            assert_close(got[g], want, "bf16", f"wgrad group {g}")


# ---- output quantisation fused into the epilogue

def _sentinel(shape):
    return torch.full(shape, 0xA5, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("sizes", [[0, 1, 17, 33, 0, 65, 129, 300, 16, 32, 64, 128, 2], [513, 0, 7]])
@pytest.mark.parametrize("epi", ["swiglu", "none"])
@pytest.mark.parametrize("fp4_in", [False, True])
def test_fused_quant_e4m3_equals_two_pass(L, sizes, epi, fp4_in):
    """GEMM with its output quantised in the epilogue (row-wise and group-aware column-wise
    MXFP8) writes the same bytes as the GEMM's bf16 output passed through the standalone dual
    quantiser: every code and scale byte, the block prefix, the untouched rows and padding;
    with C omitted the quantised copies are unchanged."""
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, G, N, K = int(off[-1]) + 3, len(sizes), 256, 512
    nb = 2 * N if epi == "swiglu" else N
    x = mi.randn_np(31, mi.X, 0, M + 4, K, 1.0, "bf16").astype(np.float64)
    W = np.stack([mi.randn_np(31, mi.W_GATE, g, nb, K, 0.05, "bf16") for g in range(G)]).astype(np.float64)
    if fp4_in:
        from tests.test_gpu_mx4 import pack
        A, As, _ = O.mx4_quantize_rowwise(x)
        parts = [O.mx4_quantize_rowwise(W[g]) for g in range(G)]
        A = pack(A)
        B = np.stack([pack(p[0]) for p in parts])
    else:
        A, As, _ = O.mx_quantize_rowwise(x)
        parts = [O.mx_quantize_rowwise(W[g]) for g in range(G)]
        B = np.stack([p[0] for p in parts])
    Bs = np.stack([p[1] for p in parts])
    a_rows = np.random.Generator(np.random.PCG64(5)).integers(0, M + 4, M).astype(np.int32)
    e = L.MOE_EPI_SWIGLU if epi == "swiglu" else L.MOE_EPI_NONE
    offs, ar = dev_i32(off), dev_i32(a_rows)
    cap = L.quant_col_blocks(M, G)
    # two-pass: bf16 output, then the dual quantiser
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.moe_grouped_gemm(_u8(A), _u8(B), C, offs, e, a_rows=ar, workspace=_ws(L, G), a_scale=_u8(As),
                       b_scale=_u8(Bs), fp4=fp4_in)
    q2, s2, qc2, sc2 = _sentinel((M, N)), _sentinel((M, N // 32)), _sentinel((N, 32 * cap)), _sentinel((N, cap))
    bs2 = torch.full((G + 1,), -1, dtype=torch.int32, device="cuda")
    L.moe_group_quant_mxfp8_dual(C, q2, s2, qc2, sc2, offs, block_start=bs2, rows=int(off[-1]))
    outs = []
    for keep_c in (True, False):
        Cf = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda") if keep_c else None
        q1, s1, qc1, sc1 = _sentinel((M, N)), _sentinel((M, N // 32)), _sentinel((N, 32 * cap)), _sentinel((N, cap))
        bs1 = torch.full((G + 1,), -1, dtype=torch.int32, device="cuda")
        L.moe_grouped_gemm(_u8(A), _u8(B), Cf, offs, e, a_rows=ar, workspace=_ws(L, G), a_scale=_u8(As),
                           b_scale=_u8(Bs), fp4=fp4_in, q_row=q1, s_row=s1, q_col=qc1, s_col=sc1, q_block_start=bs1,
                           out_shape=(M, N))
        torch.cuda.synchronize()
        if keep_c:
            np.testing.assert_array_equal(bits(Cf), bits(C))
        outs.append([t.cpu().numpy() for t in (q1, s1, qc1, sc1, bs1)])
    torch.cuda.synchronize()
    want = [t.cpu().numpy() for t in (q2, s2, qc2, sc2, bs2)]
    for got in outs:
        for name, a, b in zip(("q_row", "s_row", "q_col", "s_col", "block_start"), got, want):
            np.testing.assert_array_equal(a, b, err_msg=name)
    assert np.all(outs[0][0][off[-1]:] == 0xA5), "rows outside the groups are not written"


def test_fused_quant_e2m1_equals_two_pass(L):
    """MXFP4 output quantisation in the epilogue equals moe_group_quant_mxfp4 on the bf16 output."""
    from tests.test_gpu_mx4 import pack
    sizes = [0, 1, 17, 33, 65, 129, 300, 2, 128, 513]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, G, N, K = int(off[-1]) + 2, len(sizes), 384, 1024
    x = mi.randn_np(33, mi.X, 0, M, K, 1.0, "bf16").astype(np.float64)
    W = np.stack([mi.randn_np(33, mi.W_GATE, g, 2 * N, K, 0.05, "bf16") for g in range(G)]).astype(np.float64)
    A, As, _ = O.mx4_quantize_rowwise(x)
    parts = [O.mx4_quantize_rowwise(W[g]) for g in range(G)]
    B = np.stack([pack(p[0]) for p in parts])
    Bs = np.stack([p[1] for p in parts])
    offs = dev_i32(off)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.moe_grouped_gemm(_u8(pack(A)), _u8(B), C, offs, L.MOE_EPI_SWIGLU, workspace=_ws(L, G), a_scale=_u8(As),
                       b_scale=_u8(Bs), fp4=True)
    q2, s2 = _sentinel((M, N // 2)), _sentinel((M, N // 32))
    L.moe_group_quant_mxfp4(C[:int(off[-1])], q2[:int(off[-1])], s2[:int(off[-1])])
    q1, s1 = _sentinel((M, N // 2)), _sentinel((M, N // 32))
    L.moe_grouped_gemm(_u8(pack(A)), _u8(B), None, offs, L.MOE_EPI_SWIGLU, workspace=_ws(L, G), a_scale=_u8(As),
                       b_scale=_u8(Bs), fp4=True, q_row=q1, s_row=s1, q_fp4=True, out_shape=(M, N))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q1.cpu().numpy(), q2.cpu().numpy())
    np.testing.assert_array_equal(s1.cpu().numpy(), s2.cpu().numpy())


@pytest.mark.parametrize("sizes", [[0, 1, 17, 33, 0, 65, 129, 300, 16, 32, 64, 128, 2], [513, 0, 7]])
@pytest.mark.parametrize("fp4_in", [False, True])
def test_swiglu_bwd_epilogue_equals_two_pass(L, sizes, fp4_in):
    """The data-gradient GEMM with the SwiGLU backward in its epilogue writes the [dg | du]
    that moe_swiglu_backward forms from the GEMM's stored bf16 dh, bit for bit, and the same
    MXFP8 copies (row-wise and column-wise over all 2N columns, block prefix) as the dual
    quantiser run on that result; with C omitted the copies are unchanged."""
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(off[-1])
    M, G, N, K = R + 3, len(sizes), 256, 512
    dy = mi.randn_np(41, mi.D_OUT, 0, M, K, 1.0, "bf16").astype(np.float64)
    W = np.stack([mi.randn_np(41, mi.W_DOWN, g, N, K, 0.05, "bf16") for g in range(G)]).astype(np.float64)
    if fp4_in:
        from tests.test_gpu_mx4 import pack
        A, As, _ = O.mx4_quantize_rowwise(dy)
        parts = [O.mx4_quantize_rowwise(W[g]) for g in range(G)]
        A = pack(A)
        B = np.stack([pack(p[0]) for p in parts])
    else:
        A, As, _ = O.mx_quantize_rowwise(dy)
        parts = [O.mx_quantize_rowwise(W[g]) for g in range(G)]
        B = np.stack([p[0] for p in parts])
    Bs = np.stack([p[1] for p in parts])
    gu = torch.from_numpy(mi.randn_np(42, mi.X, 0, M, 2 * N, 2.0, "bf16")).to(torch.bfloat16).cuda()
    offs = dev_i32(off)
    cap = L.quant_col_blocks(M, G)
    dh = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.moe_grouped_gemm(_u8(A), _u8(B), dh, offs, L.MOE_EPI_NONE, workspace=_ws(L, G), a_scale=_u8(As),
                       b_scale=_u8(Bs), fp4=fp4_in)
    dgu = torch.full((M, 2 * N), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.moe_swiglu_backward(dh[:R], gu[:R], dgu[:R])
    q2, s2, qc2, sc2 = (_sentinel((M, 2 * N)), _sentinel((M, 2 * N // 32)), _sentinel((2 * N, 32 * cap)),
                        _sentinel((2 * N, cap)))
    bs2 = torch.full((G + 1,), -1, dtype=torch.int32, device="cuda")
    L.moe_group_quant_mxfp8_dual(dgu, q2, s2, qc2, sc2, offs, block_start=bs2, rows=R)
    want = [t.cpu().numpy() for t in (q2, s2, qc2, sc2, bs2)]
    for keep_c in (True, False):
        C = torch.full((M, 2 * N), float("nan"), dtype=torch.bfloat16, device="cuda") if keep_c else None
        q1, s1, qc1, sc1 = (_sentinel((M, 2 * N)), _sentinel((M, 2 * N // 32)), _sentinel((2 * N, 32 * cap)),
                            _sentinel((2 * N, cap)))
        bs1 = torch.full((G + 1,), -1, dtype=torch.int32, device="cuda")
        L.moe_grouped_gemm(_u8(A), _u8(B), C, offs, L.MOE_EPI_SWIGLU_BWD, aux=gu, workspace=_ws(L, G),
                           a_scale=_u8(As), b_scale=_u8(Bs), fp4=fp4_in, q_row=q1, s_row=s1, q_col=qc1, s_col=sc1,
                           q_block_start=bs1, out_shape=(M, 2 * N))
        torch.cuda.synchronize()
        if keep_c:
            np.testing.assert_array_equal(bits(C)[:R], bits(dgu)[:R])
            assert np.all(np.isnan(host(C[R:]))), "rows outside the groups are not written"
        for name, a, b in zip(("q_row", "s_row", "q_col", "s_col", "block_start"),
                              [t.cpu().numpy() for t in (q1, s1, qc1, sc1, bs1)], want):
            np.testing.assert_array_equal(a, b, err_msg=name)
