"""moe_grouped_gemm on the GPU vs the oracle.

Exactly representable inputs make the fp32 result exact whatever the summation order, so
every element must match bit for bit: this pins tile placement, row/column masking,
the gather index and the group schedule across every tile height. Random bf16 inputs
check the SwiGLU epilogue and its saved pre-activations within tolerance, and the
DeepSeek-V3-shaped launch is checked on sampled rows of sampled experts."""
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


def _ws(L, G):
    return torch.empty((L.moe_workspace_bytes(L.MOE_OP_GROUPED_GEMM, 0, 0, 0, 0, G),), dtype=torch.uint8,
                       device="cuda")


def _gemm(L, A, B, offsets, M, N, epi, c_dtype, a_rows=None, aux=False):
    C = torch.full((M, N), float("nan"), dtype=c_dtype, device="cuda")
    X = torch.full((M, 2 * N), float("nan"), dtype=c_dtype, device="cuda") if aux else None
    L.moe_grouped_gemm(A, B, C, dev_i32(offsets), epi, a_rows=None if a_rows is None else dev_i32(a_rows), aux=X,
                       workspace=_ws(L, B.shape[0]))
    torch.cuda.synchronize()
    return C, X


SIZES = [[0, 1, 17, 33, 0, 65, 129, 300, 16, 32, 64, 128, 2],   # every tile height, empty groups
         [513], [0, 0, 5]]


@pytest.mark.parametrize("sizes", SIZES)
@pytest.mark.parametrize("N,K", [(256, 512), (192, 128), (520, 64)])
@pytest.mark.parametrize("gather", [False, True])
def test_grouped_gemm_integer_exact(L, sizes, N, K, gather):
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(off[-1]) + 3                          # rows past offsets[G] must stay untouched
    G = len(sizes)
    A = mi.integer_valued((M + 7, K), -2, 2, 0, N + K)
    B = mi.integer_valued((G, N, K), -2, 2, -3, G)
    a_rows = np.random.Generator(np.random.PCG64(3)).integers(0, M + 7, M).astype(np.int32) if gather else None
    C, _ = _gemm(L, dev(A, "bf16"), dev(B, "bf16"), off, M, N, L.MOE_EPI_NONE, torch.float32, a_rows)
    want = O.grouped_gemm(A, B, off, a_row_index=a_rows)
    got = host(C)
    np.testing.assert_array_equal(got[:off[-1]], want)
    assert np.all(np.isnan(got[off[-1]:]))


# bf16 output: without a row index, groups' full 256-row chunks take 256 x 256 tiles and the
# rest the smaller row tiles. Integer sums below 2^24 are exact in fp32, so C is the exact sum
# rounded once to bf16.
SIZES_256 = [[300, 0, 256, 513, 1, 1024, 37, 255], [2048]]


@pytest.mark.parametrize("sizes", SIZES_256)
@pytest.mark.parametrize("N,K", [(256, 512), (264, 64), (512, 1024)])
@pytest.mark.parametrize("gather", [False, True])
def test_grouped_gemm_integer_exact_bf16_out(L, sizes, N, K, gather):
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(off[-1]) + 3
    G = len(sizes)
    A = mi.integer_valued((M + 7, K), -2, 2, 0, N + K + 1)
    B = mi.integer_valued((G, N, K), -2, 2, -3, G + 1)
    a_rows = np.random.Generator(np.random.PCG64(4)).integers(0, M + 7, M).astype(np.int32) if gather else None
    C, _ = _gemm(L, dev(A, "bf16"), dev(B, "bf16"), off, M, N, L.MOE_EPI_NONE, torch.bfloat16, a_rows)
    want = O.grouped_gemm(A, B, off, a_row_index=a_rows, rnd=O.round_bf16)
    got = host(C)
    np.testing.assert_array_equal(got[:off[-1]], want)
    assert np.all(np.isnan(got[off[-1]:]))


def _split_rows(off, cap=255):
    """The same rows cut into groups of at most `cap` rows, and each piece's parent group."""
    new, parent = [0], []
    for g in range(len(off) - 1):
        r = int(off[g])
        while r < off[g + 1]:
            r = min(r + cap, int(off[g + 1]))
            new.append(r)
            parent.append(g)
    return np.array(new, np.int32), np.array(parent, np.int64)


@pytest.mark.parametrize("epi", ["none", "swiglu"])
@pytest.mark.parametrize("N,K", [(384, 1024), (200, 192)])
def test_split256_bit_identical_to_128_row_tiles(L, epi, N, K):
    """256 x 256 tiles run the 128-row tiles' K order and MFMA: the same rows cut into groups
    below 256 rows (weights copied per piece, so no 256-row chunk exists) give the same bits,
    and so does the persistent kernel with load waves (SwiGLU with the G|U save)."""
    sizes = [700, 0, 256, 1, 1300, 90, 512]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, G = int(off[-1]), len(sizes)
    nb = 2 * N if epi == "swiglu" else N
    x = dev(mi.randn_np(5, mi.X, 0, M, K, 1.0, "bf16"), "bf16")
    B = dev(np.stack([mi.randn_np(5, mi.W_GATE, g, nb, K, 0.05, "bf16") for g in range(G)]), "bf16")
    a_rows = None                                        # a row index turns the split off
    e = L.MOE_EPI_SWIGLU if epi == "swiglu" else L.MOE_EPI_NONE
    C1, _ = _gemm(L, x, B, off, M, N, e, torch.bfloat16, a_rows)
    off2, parent = _split_rows(off)
    B2 = B[torch.from_numpy(parent).cuda()].contiguous()
    C2, _ = _gemm(L, x, B2, off2, M, N, e, torch.bfloat16, a_rows)
    np.testing.assert_array_equal(bits(C1), bits(C2))
    if epi == "swiglu":
        # with the G|U save the launch does not split: the persistent kernel with load waves
        C3, _ = _gemm(L, x, B, off, M, N, e, torch.bfloat16, a_rows, aux=True)
        np.testing.assert_array_equal(bits(C1), bits(C3))


def test_split256_full_size_down_projection_bit_identical(L):
    """DeepSeek-V3-shaped down projection (the layer's GEMM 2: 257 groups, 73,728 rows,
    d = 7168, f = 2048) with its 256-row chunks on 256 x 256 tiles, against the same rows cut
    into groups below 256 rows: every one of the 528M outputs bit-identical."""
    import os
    w = mi.WORKLOADS["dsv3"]
    with open(os.path.join(os.path.dirname(__file__), "golden", "offsets_dsv3.txt")) as fh:
        off = np.array([int(v) for v in [ln for ln in fh if not ln.startswith("#")][0].split()], np.int32)
    M, G = int(off[-1]), len(off) - 1
    gen = torch.Generator(device="cuda").manual_seed(7)
    H = torch.randn((M, w.f), generator=gen, device="cuda").to(torch.bfloat16)
    W = (torch.randn((G, w.d, w.f), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    C1, _ = _gemm(L, H, W, off, M, w.d, L.MOE_EPI_NONE, torch.bfloat16)
    off2, parent = _split_rows(off)
    W2 = W[torch.from_numpy(parent).cuda()].contiguous()
    del W
    C2, _ = _gemm(L, H, W2, off2, M, w.d, L.MOE_EPI_NONE, torch.bfloat16)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    assert not torch.isnan(C1).any()


@pytest.mark.parametrize("sizes,N,K", [([40, 0, 1, 200, 7, 129], 384, 256), ([1000], 128, 320)])
def test_grouped_swiglu_bf16(L, sizes, N, K):
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, G = int(off[-1]), len(sizes)
    A = mi.randn_np(1, mi.X, 0, M, K, 1.0, "bf16")
    B = np.stack([mi.randn_np(1, mi.W_GATE, g, 2 * N, K, 0.05, "bf16") for g in range(G)])
    H, GU = _gemm(L, dev(A, "bf16"), dev(B, "bf16"), off, M, N, L.MOE_EPI_SWIGLU, torch.bfloat16, aux=True)
    want = O.grouped_swiglu(A, B, off, rnd=O.round_bf16)
    assert_close(host(H), want, "bf16", "H")
    # saved pre-activations: G and U rounded once to bf16
    Gm = O.grouped_gemm(A, B[:, :N], off, rnd=O.round_bf16)
    Um = O.grouped_gemm(A, B[:, N:], off, rnd=O.round_bf16)
    assert_close(host(GU)[:, :N], Gm, "bf16", "G")
    assert_close(host(GU)[:, N:], Um, "bf16", "U")


def test_grouped_swiglu_fp32(L):
    sizes = [9, 0, 40, 3]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, G, N, K = int(off[-1]), len(sizes), 256, 128
    A = mi.randn_np(2, mi.X, 0, M, K, 1.0, "f32")
    B = np.stack([mi.randn_np(2, mi.W_GATE, g, 2 * N, K, 0.02, "f32") for g in range(G)])
    H, _ = _gemm(L, dev(A, "f32"), dev(B, "f32"), off, M, N, L.MOE_EPI_SWIGLU, torch.float32)
    assert_close(host(H), O.grouped_swiglu(A, B, off, rnd=O.round_f32), "f32", "H")


def test_fused_gather_equals_materialised_gather(L):
    sizes = [300, 0, 3, 77]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, G, N, K = int(off[-1]), len(sizes), 256, 256
    x = mi.randn_np(4, mi.X, 0, 150, K, 1.0, "bf16")
    src = np.random.Generator(np.random.PCG64(8)).integers(0, 150, M).astype(np.int32)
    B = np.stack([mi.randn_np(4, mi.W_GATE, g, 2 * N, K, 0.05, "bf16") for g in range(G)])
    Bd = dev(B, "bf16")
    H1, _ = _gemm(L, dev(x, "bf16"), Bd, off, M, N, L.MOE_EPI_SWIGLU, torch.bfloat16, a_rows=src)
    H2, _ = _gemm(L, dev(x[src], "bf16"), Bd, off, M, N, L.MOE_EPI_SWIGLU, torch.bfloat16)
    np.testing.assert_array_equal(bits(H1), bits(H2))


def test_grouped_gemm_dsv3_shape_integer_exact_sampled(L):
    """The DeepSeek-V3 gate/up launch shape (257 groups with the workload's real skew,
    K = 7168, 2f = 4096 columns) on exactly representable inputs, fp32 output; sampled rows
    of the hottest, a median, a tiny and the shared group must match exactly."""
    w = mi.WORKLOADS["dsv3"]
    idx, _, _ = O.route(mi.x_np(w), mi.w_router_np(w), mi.expert_bias(w), w.k, w.score)
    off, _, src = O.permutation(idx, w.E, w.T)
    M, G, N, K = int(off[-1]), w.E + 1, 2 * w.f, w.d
    x = mi.integer_valued((w.T, K), -2, 2, 0, 31)
    Bd = torch.empty((G, N, K), dtype=torch.bfloat16, device="cuda")
    for g in range(G):                                  # same values as randint_np, made on the device
        mi.randint_torch(77, mi.W_GATE, g, N, K, -2, 2, -3, "bf16", "cuda", out=Bd[g])
    C, _ = _gemm(L, dev(x, "bf16"), Bd, off, M, N, L.MOE_EPI_NONE, torch.float32, a_rows=src)
    del Bd
    counts = np.diff(off)
    picks = {int(np.argmax(counts[:w.E])), int(np.argsort(counts[:w.E])[w.E // 2]),
             int(np.argmin(np.where(counts[:w.E] > 0, counts[:w.E], 1 << 30))), w.E}
    rng = np.random.Generator(np.random.PCG64(0))
    for g in sorted(picks):
        lo, hi = int(off[g]), int(off[g + 1])
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, 24)]))
        Bg = mi.randint_np(77, mi.W_GATE, g, N, K, -2, 2, -3).astype(np.float64)
        want = x[src[rows]].astype(np.float64) @ Bg.T
        got = C[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
        np.testing.assert_array_equal(got, want, err_msg=f"group {g}")
