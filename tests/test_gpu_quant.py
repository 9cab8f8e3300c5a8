"""moe_group_quant_mxfp8 on the GPU vs the oracle: E4M3 codes and E8M0 scale bytes must match
bit for bit (the quantiser is a deterministic function), row-wise and group-aware
column-wise, including saturating blocks, all-zero and signed-zero blocks, partial, empty
and one-row groups, rows read through a gather index, and sampled rows/columns at the
DeepSeek-V3 shapes. In the column-wise layout every group starts on a multiple of four
blocks; the blocks between a group's last row and the next group are checked to be zero."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as O
from tests.gpu_util import dev, dev_i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    from dropless_mixture_experts_device_amd import _lib
    return _lib


def _nasty(rows, cols, seed, dtype="bf16"):
    """bf16-exact values with a different power-of-two range per row, plus special blocks."""
    a = mi.randn_np(seed, mi.X, 0, rows, cols, 1.0, dtype).astype(np.float64)
    g = np.random.Generator(np.random.PCG64(seed))
    a *= np.ldexp(1.0, g.integers(-20, 21, rows))[:, None]
    if rows >= 4 and cols >= 64:
        a[0, :32] = 0.0                                  # all-zero block
        a[1, :32] = -0.0                                 # signed zeros
        a[2, 5] = 1.875 * 2.0 ** 3                       # amax mantissa 1.875 -> 448 saturation
        a[2, :32] = np.clip(a[2, :32], -15.0, 15.0)
        a[2, 5] = 1.875 * 2.0 ** 3
        a[3, 32:64] = 2.0 ** -7                          # constant block on an exact power of two
    return a


def _rowwise(L, a, dtype="bf16"):
    x = dev(a, dtype)
    rows, cols = a.shape
    q = torch.full((rows, cols), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((rows, cols // 32), 0xAB, dtype=torch.uint8, device="cuda")
    L.moe_group_quant_mxfp8(x, q, s, axis=0)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("rows,cols,dtype", [(64, 128, "bf16"), (300, 7168, "bf16"), (7, 32, "bf16"),
                                             (50, 96, "f32")])
def test_quant_rowwise_bit_exact(L, rows, cols, dtype):
    a = _nasty(rows, cols, rows + cols, dtype)
    q, s = _rowwise(L, a, dtype)
    wq, ws, _ = O.mx_quantize_rowwise(a)
    np.testing.assert_array_equal(s, ws)
    np.testing.assert_array_equal(q, wq)


def _colwise(L, a, offsets, dtype="bf16", row_index=None):
    """Column-wise quantisation of a (or of a[row_index] read through the gather)."""
    G = len(offsets) - 1
    rows = a.shape[0] if row_index is None else len(row_index)
    cols = a.shape[1]
    nblk = L.quant_col_blocks(rows, G)
    x = dev(a, dtype)
    q = torch.full((cols, 32 * nblk), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((cols, nblk), 0xAB, dtype=torch.uint8, device="cuda")
    bs = torch.full((G + 1,), -1, dtype=torch.int32, device="cuda")
    L.moe_group_quant_mxfp8(x, q, s, axis=1, group_offsets=dev_i32(offsets), block_start=bs,
                            row_index=None if row_index is None else dev_i32(row_index))
    torch.cuda.synchronize()
    return q.cpu().numpy().reshape(-1), s.cpu().numpy().reshape(-1), bs.cpu().numpy()


def _group_blocks(qf, sf, bs, cols, g):
    """Group g's transposed block of the group-major layout: codes [cols, 32 n_g] starting at
    byte 32*cols*block_start[g], scales [cols, n_g] at cols*block_start[g]."""
    b0, b1 = int(bs[g]), int(bs[g + 1])
    return (qf[32 * cols * b0:32 * cols * b1].reshape(cols, 32 * (b1 - b0)),
            sf[cols * b0:cols * b1].reshape(cols, b1 - b0))


def _check_colwise(a, offsets, qf, sf, bs, cols=None, col_subset=None):
    """a: the input columns checked ([rows, len(col_subset)] when a subset is given)."""
    off = np.asarray(offsets, np.int64)
    nb = 4 * (-(-np.diff(off) // 128))
    np.testing.assert_array_equal(bs, np.concatenate([[0], np.cumsum(nb)]))
    cols = a.shape[1] if cols is None else cols
    sel = np.arange(cols) if col_subset is None else np.asarray(col_subset)
    codes, scales, _ = O.mx_quantize_colwise_grouped(a, off)
    for g in range(len(off) - 1):
        lo, hi = int(off[g]), int(off[g + 1])
        m = hi - lo
        qg, sg = _group_blocks(qf, sf, bs, cols, g)
        qg, sg = qg[sel], sg[sel]
        for i in range(int(nb[g])):
            blk = qg[:, 32 * i:32 * i + 32]
            if 32 * i >= m:      # alignment block past the group's rows
                assert np.all(sg[:, i] == 0) and np.all(blk == 0), f"group {g} block {i} must be all zero"
                continue
            n = min(32, m - 32 * i)
            np.testing.assert_array_equal(sg[:, i], scales[g][i], err_msg=f"group {g} block {i}")
            np.testing.assert_array_equal(blk[:, :n], codes[lo + 32 * i:lo + 32 * i + n].T)
            assert np.all(blk[:, n:] == 0), "padding rows of a partial block must be zero codes"


@pytest.mark.parametrize("sizes,cols,dtype", [([0, 1, 33, 0, 100, 64, 31], 96, "bf16"), ([5], 64, "bf16"),
                                              ([300, 0, 0], 320, "bf16"), ([0, 1, 33, 0, 200, 64, 31], 200, "f32")])
def test_quant_colwise_grouped_bit_exact(L, sizes, cols, dtype):
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    a = _nasty(int(off[-1]), cols, cols + len(sizes), dtype)
    q, s, bs = _colwise(L, a, off, dtype)
    _check_colwise(a, off, q, s, bs)


def test_quant_gather_rows_bit_exact(L):
    """row_index reads logical row r from x[row_index[r]] in both layouts (repeats included)."""
    a = _nasty(90, 96, 4)
    ri = np.random.Generator(np.random.PCG64(6)).integers(0, 90, 200).astype(np.int32)
    x = dev(a, "bf16")
    q = torch.full((200, 96), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((200, 3), 0xAB, dtype=torch.uint8, device="cuda")
    L.moe_group_quant_mxfp8(x, q, s, axis=0, row_index=dev_i32(ri))
    torch.cuda.synchronize()
    wq, ws, _ = O.mx_quantize_rowwise(a[ri])
    np.testing.assert_array_equal(s.cpu().numpy(), ws)
    np.testing.assert_array_equal(q.cpu().numpy(), wq)
    off = np.array([0, 70, 70, 71, 200], np.int32)
    qc, sc, bs = _colwise(L, a, off, row_index=ri)
    _check_colwise(a[ri], off, qc, sc, bs)


def test_quant_dsv3_shapes_sampled(L):
    """Row-wise quantisation of a [73728, 7168] activation and group-wise column quantisation
    with the DeepSeek-V3 routing's 257 groups, checked on sampled rows and columns."""
    w = mi.WORKLOADS["dsv3"]
    idx, _, _ = O.route(mi.x_np(w), mi.w_router_np(w), mi.expert_bias(w), w.k, w.score)
    off, _, _ = O.permutation(idx, w.E, w.T)
    rows, cols = int(off[-1]), w.d
    x = mi.randn_torch(w.seed, mi.D_OUT, 9, rows, cols, 1.0, "bf16", "cuda")
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    L.moe_group_quant_mxfp8(x, q, s, axis=0)
    G = len(off) - 1
    nblk = L.quant_col_blocks(rows, G)
    qc = torch.empty((cols, 32 * nblk), dtype=torch.uint8, device="cuda")
    sc = torch.empty((cols, nblk), dtype=torch.uint8, device="cuda")
    bs = torch.empty((G + 1,), dtype=torch.int32, device="cuda")
    L.moe_group_quant_mxfp8(x, qc, sc, axis=1, group_offsets=dev_i32(off), block_start=bs)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(5))
    r_s = np.unique(np.concatenate([[0, rows - 1], rng.integers(0, rows, 30)]))
    a_rows = mi.randn_np(w.seed, mi.D_OUT, 9, r_s, cols, 1.0, "bf16").astype(np.float64)
    wq, ws, _ = O.mx_quantize_rowwise(a_rows)
    rs_t = torch.from_numpy(r_s).cuda()
    np.testing.assert_array_equal(s[rs_t].cpu().numpy(), ws)
    np.testing.assert_array_equal(q[rs_t].cpu().numpy(), wq)
    c_s = np.unique(np.concatenate([[0, cols - 1], rng.integers(0, cols, 6)]))
    full_cols = mi.randn_np(w.seed, mi.D_OUT, 9, rows, cols, 1.0, "bf16", col_index=c_s).astype(np.float64)
    _check_colwise(full_cols, off, qc.cpu().numpy().reshape(-1), sc.cpu().numpy().reshape(-1), bs.cpu().numpy(),
                   cols=cols, col_subset=c_s)


def _rounding_sweep():
    """Blocks of 32 whose maximum is 1.0 (scale byte 119: values are multiplied by 2^8 before
    rounding), the other 31 elements sweeping every E4M3 rounding case: the subnormal range
    in half-quantum steps (ties between subnormal codes included), and in every normal
    binade the midpoints between adjacent codes and the bf16 values just either side of
    them, in both signs. All values are exact in bf16."""
    vals = [k * 2.0 ** -18 for k in range(0, 17)]                       # scaled k * 2^-10: subnormals
    for e in range(-6, 8):
        for m in range(8):
            for d in (-1, 0, 1):
                vals.append((1.0 + (2 * m + 1) / 16.0 + d / 128.0) * 2.0 ** (e - 8))
    vals = [v for v in vals if v <= 1.0]
    vals = np.array(vals + [-v for v in vals])
    n_rows = -(-len(vals) // 31)
    n_rows += (-n_rows) % 8                                              # columns of the transpose: 16-byte rows
    a = np.zeros((n_rows, 32))
    a[:, 0] = 1.0
    flat = a[:, 1:].reshape(-1)
    flat[:len(vals)] = vals
    a[:, 1:] = flat.reshape(n_rows, 31)
    return a


def test_quant_rounding_sweep_bit_exact(L):
    a = _rounding_sweep()
    q, s = _rowwise(L, a)
    wq, ws, _ = O.mx_quantize_rowwise(a)
    np.testing.assert_array_equal(s, ws)
    np.testing.assert_array_equal(q, wq)
    at = np.ascontiguousarray(a.T)                                       # the same blocks, column-wise
    off = np.array([0, 32], np.int32)
    qc, sc, bs = _colwise(L, at, off)
    _check_colwise(at, off, qc, sc, bs)


def _dual(L, a, offsets, dtype="bf16", row_index=None):
    """Both copies from moe_group_quant_mxfp8_dual, sentinel-filled so unwritten bytes show."""
    G = len(offsets) - 1
    rows = a.shape[0] if row_index is None else len(row_index)
    cols = a.shape[1]
    nblk = L.quant_col_blocks(rows, G)
    x = dev(a, dtype)
    qr = torch.full((rows, cols), 0xAB, dtype=torch.uint8, device="cuda")
    sr = torch.full((rows, cols // 32), 0xAB, dtype=torch.uint8, device="cuda")
    qc = torch.full((cols, 32 * nblk), 0xAB, dtype=torch.uint8, device="cuda")
    sc = torch.full((cols, nblk), 0xAB, dtype=torch.uint8, device="cuda")
    bs = torch.full((G + 1,), -1, dtype=torch.int32, device="cuda")
    L.moe_group_quant_mxfp8_dual(x, qr, sr, qc, sc, dev_i32(offsets), block_start=bs,
                                 row_index=None if row_index is None else dev_i32(row_index))
    torch.cuda.synchronize()
    return (qr.cpu().numpy(), sr.cpu().numpy(), qc.cpu().numpy().reshape(-1), sc.cpu().numpy().reshape(-1),
            bs.cpu().numpy())


@pytest.mark.parametrize("sizes,cols,dtype", [([0, 1, 33, 0, 100, 64, 31], 96, "bf16"), ([5], 64, "bf16"),
                                              ([300, 0, 0], 320, "bf16"), ([0, 1, 33, 0, 200, 64, 31], 224, "f32"),
                                              ([128, 256, 128], 160, "bf16")])
def test_quant_dual_bit_exact(L, sizes, cols, dtype):
    """Both copies of the one-pass quantiser against the oracle: row-wise codes and scales of
    every row, and the group-major column-wise layout (alignment blocks all zero)."""
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    a = _nasty(int(off[-1]), cols, 3 * cols + len(sizes), dtype)
    qr, sr, qc, sc, bs = _dual(L, a, off, dtype)
    wq, ws, _ = O.mx_quantize_rowwise(a)
    np.testing.assert_array_equal(sr, ws)
    np.testing.assert_array_equal(qr, wq)
    _check_colwise(a, off, qc, sc, bs)


def test_quant_dual_gather_matches_single_calls(L):
    """Through a row gather (repeated rows, an empty group): the dual call writes exactly the
    bytes of the two single-axis calls."""
    a = _nasty(90, 192, 8)
    ri = np.random.Generator(np.random.PCG64(9)).integers(0, 90, 333).astype(np.int32)
    off = np.array([0, 70, 70, 171, 333], np.int32)
    qr, sr, qc, sc, bs = _dual(L, a, off, row_index=ri)
    x = dev(a, "bf16")
    q1 = torch.full((333, 192), 0xAB, dtype=torch.uint8, device="cuda")
    s1 = torch.full((333, 6), 0xAB, dtype=torch.uint8, device="cuda")
    L.moe_group_quant_mxfp8(x, q1, s1, axis=0, row_index=dev_i32(ri))
    q2, s2, bs2 = _colwise(L, a, off, row_index=ri)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(qr, q1.cpu().numpy())
    np.testing.assert_array_equal(sr, s1.cpu().numpy())
    np.testing.assert_array_equal(qc, q2)
    np.testing.assert_array_equal(sc, s2)
    np.testing.assert_array_equal(bs, bs2)


def test_quant_dual_expert_weight_stack(L):
    """The layer's use on a stack of expert weights (8 groups of 2f = 4096 rows, d = 7168, the
    DeepSeek-V3 gate/up shape for 8 experts): both copies equal the single-axis calls byte for
    byte, and sampled rows / columns equal the oracle."""
    G, R, C = 8, 4096, 7168
    w = torch.empty((G * R, C), dtype=torch.bfloat16, device="cuda")
    mi.randn_torch(11, mi.X, 0, G * R, C, 0.02, "bf16", "cuda", out=w)
    off = torch.arange(G + 1, dtype=torch.int32, device="cuda") * R
    nblk = L.quant_col_blocks(G * R, G)
    qr = torch.empty((G * R, C), dtype=torch.uint8, device="cuda")
    sr = torch.empty((G * R, C // 32), dtype=torch.uint8, device="cuda")
    qc = torch.empty((C, 32 * nblk), dtype=torch.uint8, device="cuda")
    sc = torch.empty((C, nblk), dtype=torch.uint8, device="cuda")
    bs = torch.empty((G + 1,), dtype=torch.int32, device="cuda")
    L.moe_group_quant_mxfp8_dual(w, qr, sr, qc, sc, off, block_start=bs)
    q1, s1 = torch.empty_like(qr), torch.empty_like(sr)
    L.moe_group_quant_mxfp8(w, q1, s1, axis=0)
    assert torch.equal(qr, q1) and torch.equal(sr, s1)
    del q1, s1
    q2, s2 = torch.empty_like(qc), torch.empty_like(sc)
    L.moe_group_quant_mxfp8(w, q2, s2, axis=1, group_offsets=off, block_start=torch.empty_like(bs))
    used = G * R // 32                                  # blocks written; the capacity holds 4 G more
    assert torch.equal(qc.view(-1)[:32 * C * used], q2.view(-1)[:32 * C * used])
    assert torch.equal(sc.view(-1)[:C * used], s2.view(-1)[:C * used])
    assert bs.cpu().tolist() == [g * used // G for g in range(G + 1)]
    del q2, s2
    g = np.random.Generator(np.random.PCG64(12))
    rws = np.unique(np.concatenate([[0, G * R - 1], g.integers(0, G * R, 40)]))
    a_rows = mi.randn_np(11, mi.X, 0, rws, C, 0.02, "bf16")
    wq, ws, _ = O.mx_quantize_rowwise(a_rows)
    idx = torch.from_numpy(rws).cuda()
    np.testing.assert_array_equal(qr[idx].cpu().numpy(), wq)
    np.testing.assert_array_equal(sr[idx].cpu().numpy(), ws)
    cs = np.unique(np.concatenate([[0, C - 1], g.integers(0, C, 6)]))
    grp = 5
    blk = mi.randn_np(11, mi.X, 0, np.arange(grp * R, (grp + 1) * R), C, 0.02, "bf16", col_index=cs)
    codes, scales, _ = O.mx_quantize_colwise_grouped(blk, np.array([0, R]))
    qg = qc.view(-1)[32 * C * grp * (R // 32):32 * C * (grp + 1) * (R // 32)].view(C, R)
    sg = sc.view(-1)[C * grp * (R // 32):C * (grp + 1) * (R // 32)].view(C, R // 32)
    cs_t = torch.from_numpy(cs).cuda()
    np.testing.assert_array_equal(qg[cs_t].cpu().numpy(), codes.T)
    np.testing.assert_array_equal(sg[cs_t].cpu().numpy(), scales[0].T)


@pytest.mark.parametrize("sizes,f", [([0, 1, 33, 0, 500, 64, 402], 256), ([700, 0, 2048, 129, 5, 1300], 2048),
                                     ([3, 0, 130, 1], 128)])
def test_swiglu_backward_quant_fused(L, sizes, f):
    """moe_swiglu_backward_quant_mxfp8_dual writes exactly the bytes of moe_swiglu_backward
    followed by moe_group_quant_mxfp8_dual; those bytes are the oracle's quantisation of that
    gradient (row-wise and group-aware column-wise), and their decoded values agree with the
    oracle's own SwiGLU backward to the MXFP8 tolerance."""
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows, G = int(off[-1]), len(sizes)
    dh = mi.randn_np(f, mi.D_OUT, 0, rows, f, 1.0, "bf16")
    gu = mi.randn_np(f, mi.D_OUT, 1, rows, 2 * f, 2.0, "bf16")
    dh_d, gu_d = dev(dh, "bf16"), dev(gu, "bf16")
    nblk = L.quant_col_blocks(rows, G)

    def bufs():
        return (torch.full((rows, 2 * f), 0xAB, dtype=torch.uint8, device="cuda"),
                torch.full((rows, 2 * f // 32), 0xAB, dtype=torch.uint8, device="cuda"),
                torch.full((2 * f, 32 * nblk), 0xAB, dtype=torch.uint8, device="cuda"),
                torch.full((2 * f, nblk), 0xAB, dtype=torch.uint8, device="cuda"),
                torch.full((G + 1,), -1, dtype=torch.int32, device="cuda"))

    fused, two = bufs(), bufs()
    L.moe_swiglu_backward_quant_mxfp8_dual(dh_d, gu_d, *fused[:4], dev_i32(off), block_start=fused[4])
    dgu = torch.empty((rows, 2 * f), dtype=torch.bfloat16, device="cuda")
    L.moe_swiglu_backward(dh_d, gu_d, dgu)
    L.moe_group_quant_mxfp8_dual(dgu, *two[:4], dev_i32(off), block_start=two[4])
    torch.cuda.synchronize()
    fb, tb = [t.cpu().numpy() for t in fused], [t.cpu().numpy() for t in two]
    for a, b, n in zip(fb, tb, ("q_row", "s_row", "q_col", "s_col", "block_start")):
        np.testing.assert_array_equal(a, b, err_msg=n)
    # the oracle's quantisation of that gradient, bit for bit
    g_gpu = dgu.float().cpu().numpy().astype(np.float64)
    wq, ws, _ = O.mx_quantize_rowwise(g_gpu)
    np.testing.assert_array_equal(fb[0], wq)
    np.testing.assert_array_equal(fb[1], ws)
    _check_colwise(g_gpu, off, fb[2].reshape(-1), fb[3].reshape(-1), fb[4])
    # decoded row-wise values against the oracle's own SwiGLU backward, quantised the same way
    G_, U_ = gu[:, :f].astype(np.float64), gu[:, f:].astype(np.float64)
    dh64 = dh.astype(np.float64)
    ref = np.concatenate([O.round_bf16(dh64 * U_ * O.silu_grad(G_)), O.round_bf16(dh64 * O.silu(G_))], 1)
    # (the GPU forms dgu in fp32, the oracle in fp64: where the two bf16 roundings differ by an
    # ulp the E4M3 code can move one step, at most 2**-3 of that element; the mean stays tiny)
    dec = O.e4m3_decode(fb[0]) * np.ldexp(1.0, fb[1].astype(np.int64) - 127).repeat(32, axis=1)
    from tests.gpu_util import rel_err
    mx, mean = rel_err(dec, O.mx_q_rows(ref))
    assert mx <= 0.125 and mean <= 1e-5, f"decoded dgu: max rel {mx:.3e} mean rel {mean:.3e}"


@pytest.mark.parametrize("T,d,E,k,shared,dtype", [(300, 256, 8, 2, True, "bf16"), (777, 320, 24, 6, False, "bf16"),
                                                  (129, 96, 5, 3, True, "f32"), (1, 64, 4, 4, True, "bf16")])
def test_combine_backward_quant_fused(L, T, d, E, k, shared, dtype):
    """moe_combine_backward_quant_mxfp8_dual writes exactly the bytes of moe_combine_backward
    (dY) followed by moe_group_quant_mxfp8_dual(dY), and those are the oracle's quantisation
    of the oracle's own dY (one rounding of each exact product, so bit-exact on both sides)."""
    g = np.random.Generator(np.random.PCG64(T + d + k))
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    wt = g.random((T, k)).astype(np.float32) + np.float32(0.05)
    wt /= wt.sum(1, keepdims=True)
    off, row_of, src = O.permutation(idx, E, shared_rows=T if shared else 0)
    rows, G, tk = int(off[-1]), len(off) - 1, T * k
    d_out = mi.randn_np(d, mi.D_OUT, 0, T, d, 1.0, dtype)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d_out_d, wt_d, ro_d, src_d, off_d = dev(d_out, dtype), torch.from_numpy(wt).cuda(), dev_i32(row_of), dev_i32(src), \
        dev_i32(off)
    nblk = L.quant_col_blocks(rows, G)

    def bufs():
        return (torch.full((rows, d), 0xAB, dtype=torch.uint8, device="cuda"),
                torch.full((rows, d // 32), 0xAB, dtype=torch.uint8, device="cuda"),
                torch.full((d, 32 * nblk), 0xAB, dtype=torch.uint8, device="cuda"),
                torch.full((d, nblk), 0xAB, dtype=torch.uint8, device="cuda"),
                torch.full((G + 1,), -1, dtype=torch.int32, device="cuda"))

    fused, two = bufs(), bufs()
    ws = torch.empty((L.moe_workspace_bytes(L.MOE_OP_COMBINE_BWD_QUANT, T, 0, 0, k, G),), dtype=torch.uint8,
                     device="cuda")
    L.moe_combine_backward_quant_mxfp8_dual(d_out_d, wt_d, ro_d, src_d, shared, *fused[:4], off_d, block_start=fused[4],
                                            workspace=ws)
    dY = torch.full((rows, d), float("nan"), dtype=dt, device="cuda")
    L.moe_combine_backward(d_out_d, wt_d, ro_d, dY[:tk], dy_shared=dY[tk:] if shared else None)
    L.moe_group_quant_mxfp8_dual(dY, *two[:4], off_d, block_start=two[4])
    torch.cuda.synchronize()
    fb, tb = [t.cpu().numpy() for t in fused], [t.cpu().numpy() for t in two]
    for a, b, n in zip(fb, tb, ("q_row", "s_row", "q_col", "s_col", "block_start")):
        np.testing.assert_array_equal(a, b, err_msg=n)
    rnd = O.round_bf16 if dtype == "bf16" else O.round_f32
    dY_ref, _ = O.combine_backward(d_out, np.zeros((tk, d)), wt, row_of, rnd)
    if shared:
        dY_ref = np.concatenate([dY_ref, rnd(d_out.astype(np.float64))], axis=0)
    wq, wsc, _ = O.mx_quantize_rowwise(dY_ref)
    np.testing.assert_array_equal(fb[0], wq)
    np.testing.assert_array_equal(fb[1], wsc)
    _check_colwise(dY_ref, off, fb[2].reshape(-1), fb[3].reshape(-1), fb[4])
