"""CPU replay of the grouped GEMM's index math on the launches the GPU path makes: every
DMA read inside its buffer (A through the gather index, the group's B rows, MXFP8 scales),
every LDS fill inside its stage, every output element of every group written exactly once,
no row outside the groups touched. Covers the full-size layer workloads (group offsets from
tests/golden, written by the oracle), the router's K-split projection, the shapes of the
GPU GEMM tests, and a seeded fuzz of ragged group layouts (empty groups, single rows, sizes
that are not multiples of 32, up to 300 groups)."""
import os

import numpy as np
import pytest

import moe_inputs as mi
from tests.gemm_replay import Launch, check_launch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _offsets(name):
    with open(os.path.join(GOLDEN, f"offsets_{name}.txt")) as f:
        lines = [ln for ln in f if not ln.startswith("#")]
    return np.array([int(v) for v in lines[0].split()], np.int64)


def _gemm1(w, off, mx=False, fp4=False):
    """GEMM 1 (gate/up + SwiGLU) as layer.py launches it: A = x [T, d] through src_token, B =
    W_gu [G, 2f, d] (MXFP8 / MXFP4: the row-wise codes and scales), C = H [rows, f]."""
    G = len(off) - 1
    rows = int(off[-1])
    mx = mx or fp4
    eb = 0.5 if fp4 else 1 if mx else 2
    a_rows = np.arange(rows, dtype=np.int64) % w.T      # any in-range gather index
    return Launch(offsets=off, M=rows, N=w.f, K=w.d, A_rows=w.T, lda=w.d, a_rows=a_rows, b_groups=G,
                  ldb=w.d, b_stride=2 * w.f * w.d, b_bytes=int(G * 2 * w.f * w.d * eb), ldc=w.f, c_esize=2,
                  swiglu=True, mx=mx, fp4=fp4, lda_scale=w.d // 32, ldb_scale=w.d // 32,
                  b_scale_stride=2 * w.f * w.d // 32, b_scale_bytes=G * 2 * w.f * w.d // 32,
                  aux_ld=2 * w.f if mx else 0)


def _gemm2(w, off, mx=False, fp4=False):
    """GEMM 2 (down): A = H [rows, f], B = W_down [G, d, f], C = Y [rows, d]."""
    G = len(off) - 1
    rows = int(off[-1])
    mx = mx or fp4
    eb = 0.5 if fp4 else 1 if mx else 2
    return Launch(offsets=off, M=rows, N=w.d, K=w.f, A_rows=rows, lda=w.f, a_rows=None, b_groups=G, ldb=w.f,
                  b_stride=w.d * w.f, b_bytes=int(G * w.d * w.f * eb), ldc=w.d, c_esize=2, swiglu=False, mx=mx,
                  fp4=fp4, lda_scale=w.f // 32, ldb_scale=w.f // 32, b_scale_stride=w.d * w.f // 32,
                  b_scale_bytes=G * w.d * w.f // 32)


def _dgrad(w, off, which):
    """The MXFP8 data-gradient GEMMs on the transposed weight copies: dgrad 2 (dH = dY W_down,
    B = [G, f, d]) and dgrad 1 (dX_perm = dGU W_gu, B = [G, d, 2f])."""
    G = len(off) - 1
    rows = int(off[-1])
    if which == 2:
        N, K = w.f, w.d
    else:
        N, K = w.d, 2 * w.f
    return Launch(offsets=off, M=rows, N=N, K=K, A_rows=rows, lda=K, a_rows=None, b_groups=G, ldb=K,
                  b_stride=N * K, b_bytes=G * N * K, ldc=N, c_esize=2, swiglu=False, mx=True, lda_scale=K // 32,
                  ldb_scale=K // 32, b_scale_stride=N * K // 32, b_scale_bytes=G * N * K // 32)


def _router(w):
    """The router's K-split projection: 4 uniform groups, group s multiplying the s-th quarter
    of x's columns by the same quarter of W_router's, fp32 partial logits [4 T, E]."""
    KS = 4
    return Launch(offsets=np.zeros(KS + 1, np.int64), M=KS * w.T, N=w.E, K=w.d // KS, A_rows=w.T, lda=w.d,
                  a_rows=None, b_groups=1, ldb=w.d, b_stride=w.d // KS, b_bytes=w.E * w.d * 2, ldc=w.E, c_esize=4,
                  swiglu=False, uniform_rows=w.T, a_group_stride=w.d // KS)


@pytest.mark.parametrize("name", ["dsv3", "dsv3_ep8", "mixtral", "qwen3"])
def test_replay_full_size_bf16_forward(name):
    w = mi.WORKLOADS[name]
    off = _offsets(name)
    assert len(off) == w.E + (2 if w.shared_f else 1) and off[-1] == w.T * w.k + (w.T if w.shared_f else 0)
    check_launch(_gemm1(w, off))
    check_launch(_gemm2(w, off))
    if w.E % 8 == 0 and w.d % 256 == 0:
        check_launch(_router(w))


def test_replay_full_size_mxfp8_step_gemms():
    w = mi.WORKLOADS["dsv3_mxfp8"]
    off = _offsets("dsv3")
    for la in (_gemm1(w, off, mx=True), _gemm2(w, off, mx=True), _dgrad(w, off, 2), _dgrad(w, off, 1)):
        check_launch(la)


@pytest.mark.parametrize("name", ["dsv3", "qwen3"])
def test_replay_full_size_mxfp4_forward_gemms(name):
    """E2M1 operands: 256 K values per stage, two scale dwords per row, the larger LDS ring."""
    w = mi.WORKLOADS[name]
    off = _offsets(name)
    check_launch(_gemm1(w, off, fp4=True))
    check_launch(_gemm2(w, off, fp4=True))


@pytest.mark.parametrize("name", ["small_softmax", "small_sigmoid", "small_mxfp8", "mid_mxfp8", "small_mxfp4"])
def test_replay_reduced_layer_workloads(name):
    """The GEMMs of the GPU layer tests at their reduced shapes, in each workload's format
    (bf16 forward, the MXFP8 step's four GEMMs, the MXFP4 forward)."""
    w = mi.WORKLOADS[name]
    off = _offsets(name)
    assert off[-1] == w.T * w.k + (w.T if w.shared_f else 0)
    if w.mxfp8:
        launches = [_gemm1(w, off, mx=True), _gemm2(w, off, mx=True), _dgrad(w, off, 2), _dgrad(w, off, 1)]
    else:
        launches = [_gemm1(w, off, fp4=w.mxfp4), _gemm2(w, off, fp4=w.mxfp4)]
    for la in launches:
        check_launch(la)


GPU_TEST_SIZES = [[0, 1, 17, 33, 0, 65, 129, 300, 16, 32, 64, 128, 2], [513], [0, 0, 5]]


@pytest.mark.parametrize("sizes", GPU_TEST_SIZES)
@pytest.mark.parametrize("N,K", [(256, 512), (192, 128), (520, 64)])
@pytest.mark.parametrize("gather", [False, True])
def test_replay_gpu_test_shapes(sizes, N, K, gather):
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    M = int(off[-1]) + 3
    G = len(sizes)
    a_rows = np.random.Generator(np.random.PCG64(3)).integers(0, M + 7, M) if gather else None
    check_launch(Launch(offsets=off, M=M, N=N, K=K, A_rows=M + 7, lda=K, a_rows=a_rows, b_groups=G, ldb=K,
                        b_stride=N * K, b_bytes=G * N * K * 2, ldc=N, c_esize=4, swiglu=False))


GPU_TEST_SIZES_256 = [[300, 0, 256, 513, 1, 1024, 37, 255], [2048]]


@pytest.mark.parametrize("sizes", GPU_TEST_SIZES_256)
@pytest.mark.parametrize("N,K", [(256, 512), (264, 64), (512, 1024)])
@pytest.mark.parametrize("gather", [False, True])
def test_replay_gpu_test_shapes_bf16_out(sizes, N, K, gather):
    """test_grouped_gemm_integer_exact_bf16_out's launches: bf16 C, so without a row index the
    full 256-row chunks take 256 x 256 tiles."""
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    M = int(off[-1]) + 3
    G = len(sizes)
    a_rows = np.random.Generator(np.random.PCG64(4)).integers(0, M + 7, M) if gather else None
    r = check_launch(Launch(offsets=off, M=M, N=N, K=K, A_rows=M + 7, lda=K, a_rows=a_rows, b_groups=G, ldb=K,
                            b_stride=N * K, b_bytes=G * N * K * 2, ldc=N, c_esize=2, swiglu=False))
    assert (r["tiles256"] > 0) == (not gather)


@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("N,K", [(384, 1024), (200, 192)])
def test_replay_split256_test_shapes(swiglu, N, K):
    """test_split256_bit_identical_to_128_row_tiles's two launches: the split one and the same
    rows in groups below 256 rows (nothing for gemm256_kernel)."""
    sizes = [700, 0, 256, 1, 1300, 90, 512]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    M = int(off[-1])
    T, a_rows = M, None                                  # rows in order: the launch splits
    nb = 2 * N if swiglu else N
    pieces = [0]
    for g in range(len(sizes)):
        r = int(off[g])
        while r < off[g + 1]:
            r = min(r + 255, int(off[g + 1]))
            pieces.append(r)
    for o in (off, np.array(pieces, np.int64)):
        G = len(o) - 1
        r = check_launch(Launch(offsets=o, M=M, N=N, K=K, A_rows=T, lda=K, a_rows=a_rows, b_groups=G, ldb=K,
                                b_stride=nb * K, b_bytes=G * nb * K * 2, ldc=N, c_esize=2, swiglu=swiglu))
        assert (r["tiles256"] > 0) == (o is off)
    if swiglu:   # the same launch with the G|U save: the persistent kernel with load waves
        G = len(off) - 1
        r = check_launch(Launch(offsets=off, M=M, N=N, K=K, A_rows=T, lda=K, a_rows=a_rows, b_groups=G, ldb=K,
                                b_stride=nb * K, b_bytes=G * nb * K * 2, ldc=N, c_esize=2, swiglu=True,
                                aux_ld=2 * N))
        assert r["tiles256"] == 0


def test_replay_split256_full_size_down_projection():
    """test_split256_full_size_down_projection_bit_identical's two launches: the DeepSeek-V3
    down projection split, and the same rows as 485 groups below 256 rows (no 256-row tile)."""
    w = mi.WORKLOADS["dsv3"]
    off = _offsets("dsv3")
    pieces = [0]
    for g in range(len(off) - 1):
        r = int(off[g])
        while r < off[g + 1]:
            r = min(r + 255, int(off[g + 1]))
            pieces.append(r)
    rows = int(off[-1])
    for o in (off, np.array(pieces, np.int64)):
        G = len(o) - 1
        r = check_launch(Launch(offsets=o, M=rows, N=w.d, K=w.f, A_rows=rows, lda=w.f, a_rows=None, b_groups=G,
                                ldb=w.f, b_stride=w.d * w.f, b_bytes=G * w.d * w.f * 2, ldc=w.d, c_esize=2,
                                swiglu=False))
        assert (r["tiles256"] > 0) == (o is off)


def _fuzz_sizes(g):
    G = int(g.integers(1, 301))
    kind = g.integers(0, 4, G)
    sizes = np.where(kind == 0, 0, np.where(kind == 1, g.integers(1, 33, G),
                                            np.where(kind == 2, g.integers(33, 300, G), g.integers(300, 2500, G))))
    return sizes.astype(np.int64)


@pytest.mark.parametrize("seed", range(16))
def test_replay_fuzz_ragged_groups(seed):
    """Seeded random group layouts: every tile height, empty and one-row groups, sizes not a
    multiple of 32, up to 300 groups, SwiGLU or plain, bf16 or MXFP8, with or without a gather
    (bf16 launches without the G|U save also split off the 256-row chunks)."""
    g = np.random.Generator(np.random.PCG64(1000 + seed))
    sizes = _fuzz_sizes(g)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    G = len(sizes)
    fmt = int(g.integers(0, 3))                          # bf16, MXFP8, MXFP4
    mx, fp4 = fmt > 0, fmt == 2
    swiglu = bool(g.integers(0, 2))
    N = int(g.choice([128, 256, 384, 1152] if mx else [64, 128, 136, 256, 520, 1024]))
    K = int(g.choice([256, 512, 1024, 2048] if fp4 else [128, 256, 512, 1024] if mx else [64, 128, 320, 1024]))
    extra = int(g.integers(0, 40))
    M = int(off[-1]) + extra
    gather = bool(g.integers(0, 2))
    A_rows = int(g.integers(1, 3000)) if gather else max(M, 1)
    a_rows = g.integers(-5, A_rows + 5, M) if gather else None      # out-of-range entries are clamped
    eb = 0.5 if fp4 else 1 if mx else 2
    nb = 2 * N if swiglu else N
    save = bool(g.integers(0, 2))                        # bf16 SwiGLU without the G|U save splits
    la = Launch(offsets=off, M=M, N=N, K=K, A_rows=A_rows, lda=K, a_rows=a_rows, b_groups=G, ldb=K,
                b_stride=nb * K, b_bytes=int(G * nb * K * eb), ldc=N, c_esize=2, swiglu=swiglu, mx=mx, fp4=fp4,
                lda_scale=K // 32, ldb_scale=K // 32, b_scale_stride=nb * K // 32, b_scale_bytes=G * nb * K // 32,
                aux_ld=2 * N if swiglu and (mx or save) else 0)
    if M == 0:
        return                                           # the host returns before launching anything
    check_launch(la)


def test_replay_catches_an_out_of_range_gather_without_clamp(monkeypatch):
    """The replay has teeth: with the kernel's clamp of the gather index removed from the model,
    an out-of-range index is reported."""
    import tests.gemm_replay as R
    off = np.array([0, 40], np.int64)
    la = Launch(offsets=off, M=40, N=128, K=64, A_rows=10, lda=64, a_rows=np.arange(40), b_groups=1, ldb=64,
                b_stride=128 * 64, b_bytes=128 * 64 * 2, ldc=128, c_esize=2, swiglu=False)
    monkeypatch.setattr(R.np, "clip", lambda a, lo, hi: a)
    with pytest.raises(AssertionError):
        check_launch(la)


MX4_GPU_TEST_LAUNCHES = [([0, 1, 17, 33, 65, 129, 300, 2], 256, 512, 2, 5), ([700], 192, 256, 2, 5),
                         ([5, 0, 90], 520, 2048, 2, 5), ([33, 0, 260, 1], 384, 1024, 0, 0),
                         ([40, 0, 1, 200, 7, 129, 513], 384, 1024, 0, 0)]


@pytest.mark.parametrize("sizes,N,K,extra_m,extra_a", MX4_GPU_TEST_LAUNCHES)
@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("swiglu", [False, True])
def test_replay_mx4_gpu_test_shapes(sizes, N, K, extra_m, extra_a, gather, swiglu):
    """The MXFP4 GEMM launches of the GPU tests (C rows beyond the groups, A rows beyond C's)."""
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    M = int(off[-1]) + extra_m
    A_rows = M + extra_a
    G = len(sizes)
    nb = 2 * N if swiglu else N
    a_rows = np.random.Generator(np.random.PCG64(2)).integers(0, A_rows, M) if gather else None
    check_launch(Launch(offsets=off, M=M, N=N, K=K, A_rows=A_rows, lda=K, a_rows=a_rows, b_groups=G, ldb=K,
                        b_stride=nb * K, b_bytes=G * nb * K // 2, ldc=N, c_esize=4, swiglu=swiglu, mx=True, fp4=True,
                        lda_scale=K // 32, ldb_scale=K // 32, b_scale_stride=nb * K // 32,
                        b_scale_bytes=G * nb * K // 32))


@pytest.mark.parametrize("w", [w for w in mi.fuzz_workloads() if w.dtype == "bf16"], ids=lambda w: w.name)
def test_replay_layer_sweep(w):
    """The GEMM launches of the seeded layer-shape sweep run on the GPU (group offsets from the
    oracle's routing of the same inputs, which the GPU's routing equals away from near-ties;
    the fuzz above covers arbitrary layouts): both expert GEMMs and, where the router takes
    the K-split path, its projection."""
    from oracle import moe_oracle as O
    idx, _, _ = O.route(mi.x_np(w), mi.w_router_np(w), mi.expert_bias(w), w.k, w.score)
    off, _, _ = O.permutation(idx, w.E, w.T if w.shared_f else 0)
    off = np.asarray(off, np.int64)
    check_launch(_gemm1(w, off))
    check_launch(_gemm2(w, off))
    if w.T >= 256 and w.E % 8 == 0 and w.d % 256 == 0:
        check_launch(_router(w))
