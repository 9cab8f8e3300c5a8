"""The C ABI library loads, exports every entry point the header declares, and rejects bad
arguments on the host (these calls return before touching the GPU, so they run on CPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
# MOE_LIB: the same tests against another build of the library (the host-ASan build)
LIB = os.environ.get("MOE_LIB") or os.path.join(ROOT, "dropless_mixture_experts_device_amd", "libmoe.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from dropless_mixture_experts_device_amd import build
        build()
    return ctypes.CDLL(LIB)


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"moe_route", "moe_permute", "moe_grouped_gemm", "moe_combine"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_debug_build_exports_every_symbol():
    """The MOE_DEBUG build (libmoe_debug.so, built next to libmoe.so) exports the same entry
    points and answers the same host-side argument checks."""
    path = os.path.join(ROOT, "dropless_mixture_experts_device_amd", "libmoe_debug.so")
    if not os.path.exists(path):
        pytest.skip("libmoe_debug.so is not built")
    dbg = ctypes.CDLL(path)
    for n in _declared():
        assert hasattr(dbg, n), n
    dbg.moe_combine.restype = ctypes.c_int
    fake = ctypes.c_void_p(1 << 20)
    args = [fake, 1, fake, fake, None, ctypes.c_int64(16), ctypes.c_int64(60), ctypes.c_int32(2), fake, None]
    assert dbg.moe_combine(*args) == 1          # d % 8 != 0: MOE_EINVAL, as the release build


def test_binding_covers_every_symbol():
    from dropless_mixture_experts_device_amd import _lib as L
    assert set(_declared()) == set(L.EXPORTED)
    for n in L.EXPORTED:
        assert callable(getattr(L, n))


def test_status_strings_and_workspace(lib):
    from dropless_mixture_experts_device_amd import _lib as L
    assert L.moe_status_str(0) == "MOE_OK"
    assert "invalid" in L.moe_status_str(1)
    assert L.moe_workspace_bytes(L.MOE_OP_ROUTE, 8192, 7168, 256, 8, 0) >= 4 * 8192 * 256 * 4
    assert L.moe_workspace_bytes(L.MOE_OP_ROUTE, 64, 128, 8, 2, 0) == 0
    pb = L.moe_workspace_bytes(L.MOE_OP_PERMUTE, 8192, 7168, 256, 8, 0)
    assert pb >= (8192 // 64) * 256 * 12
    assert L.moe_workspace_bytes(L.MOE_OP_GROUPED_GEMM, 0, 0, 0, 0, 257) >= 258 * 4


def test_host_argument_errors_enqueue_nothing(lib):
    from dropless_mixture_experts_device_amd import _lib as L
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: every call fails validation
    # k > E
    assert L._lib.moe_route(fake, fake, L.MOE_BF16, None, 16, 64, 4, 5, 0, fake, fake, None, None, 0, None) == L.MOE_EINVAL
    # E too large, bad score, bad dtype, d not a multiple of 8, null output
    assert L._lib.moe_route(fake, fake, L.MOE_BF16, None, 16, 64, 300, 2, 0, fake, fake, None, None, 0, None) == L.MOE_EINVAL
    assert L._lib.moe_route(fake, fake, L.MOE_BF16, None, 16, 64, 8, 2, 7, fake, fake, None, None, 0, None) == L.MOE_EINVAL
    assert L._lib.moe_route(fake, fake, L.MOE_E4M3, None, 16, 64, 8, 2, 0, fake, fake, None, None, 0, None) == L.MOE_ENOTSUP
    assert L._lib.moe_route(fake, fake, L.MOE_BF16, None, 16, 60, 8, 2, 0, fake, fake, None, None, 0, None) == L.MOE_EINVAL
    assert L._lib.moe_route(fake, fake, L.MOE_BF16, None, 16, 64, 8, 2, 0, None, fake, None, None, 0, None) == L.MOE_EINVAL
    # misaligned input
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert L._lib.moe_route(odd, fake, L.MOE_BF16, None, 16, 64, 8, 2, 0, fake, fake, None, None, 0, None) == L.MOE_EINVAL
    # a large bf16 layer needs the split-K workspace
    assert L._lib.moe_route(fake, fake, L.MOE_BF16, None, 8192, 7168, 256, 8, 1, fake, fake, None, None, 0, None) == L.MOE_EWORKSPACE
    # T == 0 is a valid no-op
    assert L._lib.moe_route(None, None, L.MOE_BF16, None, 0, 64, 8, 2, 0, None, None, None, None, 0, None) == L.MOE_OK
    # permute: workspace missing / too small / misaligned
    assert L._lib.moe_permute(None, L.MOE_BF16, fake, 64, 64, 8, 2, 0, fake, fake, fake, None, None, 0, None) == L.MOE_EWORKSPACE
    assert L._lib.moe_permute(None, L.MOE_BF16, fake, 64, 64, 8, 2, 0, fake, fake, fake, None, fake, 16, None) == L.MOE_EWORKSPACE
    assert L._lib.moe_permute(None, L.MOE_BF16, fake, 64, 64, 8, 9, 0, fake, fake, fake, None, fake, 1 << 20, None) == L.MOE_EINVAL
    # combine
    assert L._lib.moe_combine(fake, L.MOE_BF16, fake, fake, None, 16, 60, 2, fake, None) == L.MOE_EINVAL
    assert L._lib.moe_combine(fake, L.MOE_BF16, fake, None, None, 16, 64, 2, fake, None) == L.MOE_EINVAL
    # grouped GEMM
    a = L.MoeGemmArgs(G=4, offsets=fake.value, M=128, N=64, K=64, A=fake.value, a_dtype=L.MOE_BF16, lda=64,
                      A_rows=128, a_rows=None, B=fake.value, b_dtype=L.MOE_BF16, ldb=64, b_group_stride=64 * 64,
                      C=fake.value, c_dtype=L.MOE_BF16, ldc=64, epilogue=L.MOE_EPI_NONE, aux=None, ld_aux=0)
    assert L._lib.moe_grouped_gemm(ctypes.byref(a), None, 0, None) == L.MOE_EWORKSPACE
    bad = L.MoeGemmArgs.from_buffer_copy(a)
    bad.N = 60
    assert L._lib.moe_grouped_gemm(ctypes.byref(bad), fake, 1 << 20, None) == L.MOE_EINVAL
    bad = L.MoeGemmArgs.from_buffer_copy(a)
    bad.b_dtype = L.MOE_F32
    assert L._lib.moe_grouped_gemm(ctypes.byref(bad), fake, 1 << 20, None) == L.MOE_ENOTSUP
    bad = L.MoeGemmArgs.from_buffer_copy(a)
    bad.b_group_stride = -64
    assert L._lib.moe_grouped_gemm(ctypes.byref(bad), fake, 1 << 20, None) == L.MOE_EINVAL
    bad = L.MoeGemmArgs.from_buffer_copy(a)
    bad.K = 96                                   # bf16 path needs K % 64 == 0
    assert L._lib.moe_grouped_gemm(ctypes.byref(bad), fake, 1 << 20, None) == L.MOE_EINVAL
    bad = L.MoeGemmArgs.from_buffer_copy(a)
    bad.M = 0
    assert L._lib.moe_grouped_gemm(ctypes.byref(bad), fake, 1 << 20, None) == L.MOE_OK
    assert L._lib.moe_grouped_gemm(None, fake, 1 << 20, None) == L.MOE_EINVAL


def test_host_argument_errors_backward_and_quant(lib):
    from dropless_mixture_experts_device_amd import _lib as L
    fake = ctypes.c_void_p(1 << 20)
    # ragged-K GEMM: MXFP8 only, no gather, no aux, C groups must not overlap
    a = L.MoeGemmArgs(G=4, offsets=fake.value, M=128, N=64, K=512, A=fake.value, a_dtype=L.MOE_E4M3, lda=512,
                      A_rows=128, a_rows=None, B=fake.value, b_dtype=L.MOE_E4M3, ldb=512, b_group_stride=0,
                      C=fake.value, c_dtype=L.MOE_BF16, ldc=64, epilogue=L.MOE_EPI_NONE, aux=None, ld_aux=0,
                      a_scale=fake.value, lda_scale=16, b_scale=fake.value, ldb_scale=16, b_scale_group_stride=0,
                      ragged_k=1, c_group_stride=128 * 64)
    assert L._lib.moe_grouped_gemm(ctypes.byref(a), None, 0, None) == L.MOE_EWORKSPACE
    for field, value, want in (("a_dtype", L.MOE_BF16, L.MOE_ENOTSUP), ("epilogue", L.MOE_EPI_SWIGLU, L.MOE_ENOTSUP),
                               ("a_rows", fake.value, L.MOE_EINVAL), ("c_group_stride", 64 * 64, L.MOE_EINVAL),
                               ("b_group_stride", 512, L.MOE_EINVAL), ("ragged_k", 2, L.MOE_EINVAL),
                               ("K", 480, L.MOE_EINVAL), ("lda_scale", 14, L.MOE_EINVAL)):
        bad = L.MoeGemmArgs.from_buffer_copy(a)
        setattr(bad, field, value)
        if field == "a_dtype":
            bad.b_dtype = value
        assert L._lib.moe_grouped_gemm(ctypes.byref(bad), fake, 1 << 20, None) == want, field
    # combine backward: dw needs y; d % 8; T == 0 is a no-op
    assert L._lib.moe_combine_backward(fake, L.MOE_BF16, fake, fake, None, 16, 64, 2, fake, None, fake, None) == L.MOE_EINVAL
    assert L._lib.moe_combine_backward(fake, L.MOE_BF16, fake, fake, fake, 16, 60, 2, fake, None, None, None) == L.MOE_EINVAL
    assert L._lib.moe_combine_backward(fake, L.MOE_E4M3, fake, fake, fake, 16, 64, 2, fake, None, None, None) == L.MOE_ENOTSUP
    assert L._lib.moe_combine_backward(None, L.MOE_BF16, None, None, None, 0, 64, 2, None, None, None, None) == L.MOE_OK
    # router backward: sizes, score, dtype, the permutation for the weight gradient, workspace
    rb = L._lib.moe_route_backward
    wsb = L.moe_workspace_bytes(L.MOE_OP_ROUTE_BWD, 16, 64, 8, 2)
    assert wsb >= 2 * 16 * 2 * 4
    ok = (fake, fake, L.MOE_BF16, fake, fake, fake, fake, fake, fake, 16, 64, 8, 2, L.MOE_SIGMOID,
          fake, fake, 1, None, None, fake, fake, fake, wsb, None)
    for i, v, want in ((10, 60, L.MOE_EINVAL), (12, 17, L.MOE_EINVAL), (12, 0, L.MOE_EINVAL), (11, 300, L.MOE_EINVAL),
                       (11, 1, L.MOE_EINVAL),
                       (13, 2, L.MOE_EINVAL), (2, L.MOE_E4M3, L.MOE_ENOTSUP), (6, None, L.MOE_EINVAL),
                       (8, None, L.MOE_EINVAL), (7, None, L.MOE_EINVAL), (3, None, L.MOE_EINVAL),
                       (21, None, L.MOE_EWORKSPACE), (22, wsb - 1, L.MOE_EWORKSPACE), (21, fake.value + 16, L.MOE_EINVAL),
                       (18, fake, L.MOE_EINVAL), (17, fake.value + 8, L.MOE_EINVAL)):
        args = list(ok)
        args[i] = v
        assert rb(*args) == want, (i, v)
    assert rb(None, None, L.MOE_BF16, None, None, None, None, None, None, 0, 64, 8, 2, L.MOE_SOFTMAX,
              None, None, 0, None, None, None, None, fake, 256, None) == L.MOE_OK
    # fused SwiGLU backward + MXFP8: f % 128, bf16 only, leading dimensions, outputs
    fq = L._lib.moe_swiglu_backward_quant_mxfp8_dual
    okf = [fake, 256, fake, 512, L.MOE_BF16, 64, 256, fake, 2, fake, 512, fake, 16, fake, 32 * 16, fake, 16, fake,
           None, 0, None]
    for i, v, want in ((6, 192, L.MOE_EINVAL), (4, L.MOE_F32, L.MOE_ENOTSUP), (1, 128, L.MOE_EINVAL),
                       (3, 256, L.MOE_EINVAL), (9, None, L.MOE_EINVAL), (10, 256, L.MOE_EINVAL),
                       (2, None, L.MOE_EINVAL), (14, 32 * 15, L.MOE_EINVAL)):
        args = list(okf)
        args[i] = v
        assert fq(*args) == want, (i, v)
    # combine backward may skip dy (only dw wanted) ...
    assert L._lib.moe_combine_backward(None, L.MOE_BF16, None, None, None, 0, 64, 2, None, None, None, None) == L.MOE_OK
    # ... and its fused MXFP8 form: d % 32, k range, dtype, workspace, outputs
    cq = L._lib.moe_combine_backward_quant_mxfp8_dual
    wsb = L.moe_workspace_bytes(L.MOE_OP_COMBINE_BWD_QUANT, 16, 0, 0, 2, 5)
    okc = [fake, L.MOE_BF16, fake, fake, fake, 16, 64, 2, 1, fake, 5, fake, 64, fake, 2, fake, 32 * 64, fake, 64, fake,
           fake, wsb, None]
    for i, v, want in ((6, 48, L.MOE_EINVAL), (7, 17, L.MOE_EINVAL), (1, L.MOE_E4M3, L.MOE_ENOTSUP),
                       (20, None, L.MOE_EWORKSPACE), (21, wsb - 1, L.MOE_EWORKSPACE), (20, fake.value + 16, L.MOE_EINVAL),
                       (4, None, L.MOE_EINVAL), (11, None, L.MOE_EINVAL), (12, 32, L.MOE_EINVAL),
                       (16, 32 * 63, L.MOE_EINVAL), (15, None, L.MOE_EINVAL), (9, None, L.MOE_EINVAL),
                       (18, 8, L.MOE_EINVAL)):
        args = list(okc)
        args[i] = v
        assert cq(*args) == want, (i, v)
    # SwiGLU backward: f % 8, leading dimensions
    assert L._lib.moe_swiglu_backward(fake, 64, fake, 128, L.MOE_BF16, 16, 60, fake, 128, None) == L.MOE_EINVAL
    assert L._lib.moe_swiglu_backward(fake, 64, fake, 96, L.MOE_BF16, 16, 64, fake, 128, None) == L.MOE_EINVAL
    assert L._lib.moe_swiglu_backward(None, 64, None, 128, L.MOE_BF16, 0, 64, None, 128, None) == L.MOE_OK
    # quantiser: cols % 32, axis, gather without the input's row count, column-wise capacity
    q = L._lib.moe_group_quant_mxfp8
    assert q(fake, L.MOE_BF16, 64, 48, 48, None, 0, None, 0, 0, fake, 48, fake, 2, None, None, 0, None) == L.MOE_EINVAL
    assert q(fake, L.MOE_BF16, 64, 64, 64, None, 0, None, 0, 2, fake, 64, fake, 2, None, None, 0, None) == L.MOE_EINVAL
    assert q(fake, L.MOE_BF16, 64, 64, 64, fake, 0, None, 0, 0, fake, 64, fake, 2, None, None, 0, None) == L.MOE_EINVAL
    cap = L.quant_col_blocks(64, 3)
    assert cap == 4 * (1 + 3)
    assert q(fake, L.MOE_BF16, 64, 64, 64, None, 0, fake, 3, 1, fake, 32 * cap - 16, fake, cap, fake, None, 0,
             None) == L.MOE_EINVAL
    assert q(fake, L.MOE_BF16, 64, 64, 64, None, 0, fake, 3, 1, fake, 32 * cap, fake, cap, None, None, 0,
             None) == L.MOE_EWORKSPACE
    # dual quantiser: cols % 32, row-wise leading dimensions and pointers, column-wise capacity,
    # workspace; checks run before anything is enqueued
    qd = L._lib.moe_group_quant_mxfp8_dual
    assert qd(fake, L.MOE_BF16, 64, 48, 48, None, 0, fake, 3, fake, 48, fake, 2, fake, 32 * cap, fake, cap, fake,
              None, 0, None) == L.MOE_EINVAL
    assert qd(fake, L.MOE_BF16, 64, 64, 64, None, 0, fake, 3, fake, 32, fake, 2, fake, 32 * cap, fake, cap, fake,
              None, 0, None) == L.MOE_EINVAL
    assert qd(fake, L.MOE_BF16, 64, 64, 64, None, 0, fake, 3, None, 64, fake, 2, fake, 32 * cap, fake, cap, fake,
              None, 0, None) == L.MOE_EINVAL
    assert qd(fake, L.MOE_BF16, 64, 64, 64, None, 0, fake, 3, fake, 64, fake, 2, fake, 32 * cap - 32, fake, cap,
              fake, None, 0, None) == L.MOE_EINVAL
    assert qd(fake, L.MOE_BF16, 64, 64, 64, None, 0, fake, 3, fake, 64, fake, 2, fake, 32 * cap, fake, cap, None,
              None, 0, None) == L.MOE_EWORKSPACE
    assert qd(fake, L.MOE_E4M3, 64, 64, 64, None, 0, fake, 3, fake, 64, fake, 2, fake, 32 * cap, fake, cap, fake,
              None, 0, None) == L.MOE_ENOTSUP


def test_host_argument_errors_mxfp4(lib):
    """MXFP4 quantiser and E2M1 GEMM operands: every rejected argument returns its status
    before anything is enqueued."""
    from dropless_mixture_experts_device_amd import _lib as L
    fake = ctypes.c_void_p(1 << 20)
    q4 = L._lib.moe_group_quant_mxfp4
    ok = [fake, L.MOE_BF16, 64, 256, 256, None, 0, fake, 128, fake, 8, None]
    for i, v, want in ((3, 240, L.MOE_EINVAL), (4, 128, L.MOE_EINVAL), (1, L.MOE_E4M3, L.MOE_ENOTSUP),
                       (8, 112, L.MOE_EINVAL), (10, 7, L.MOE_EINVAL), (7, None, L.MOE_EINVAL),
                       (9, None, L.MOE_EINVAL), (0, None, L.MOE_EINVAL), (8, 136, L.MOE_EINVAL),
                       (7, fake.value + 8, L.MOE_EINVAL), (5, fake, L.MOE_EINVAL), (2, -1, L.MOE_EINVAL)):
        args = list(ok)
        args[i] = v
        assert q4(*args) == want, (i, v)
    # nothing to do for zero rows, even with null buffers
    assert q4(None, L.MOE_BF16, 0, 256, 256, None, 0, None, 128, None, 8, None) == L.MOE_OK
    # E2M1 GEMM: K % 256, even element strides, no ragged-K mode, at most 1023 groups (the
    # block-scaled row tiles' scale ring leaves LDS for a prefix of 1024 entries)
    a = L.MoeGemmArgs(G=4, offsets=fake.value, M=128, N=64, K=512, A=fake.value, a_dtype=L.MOE_E2M1, lda=512,
                      A_rows=128, a_rows=None, B=fake.value, b_dtype=L.MOE_E2M1, ldb=512, b_group_stride=64 * 512,
                      C=fake.value, c_dtype=L.MOE_BF16, ldc=64, epilogue=L.MOE_EPI_NONE, aux=None, ld_aux=0,
                      a_scale=fake.value, lda_scale=16, b_scale=fake.value, ldb_scale=16,
                      b_scale_group_stride=64 * 16, ragged_k=0, c_group_stride=0)
    assert L._lib.moe_grouped_gemm(ctypes.byref(a), None, 0, None) == L.MOE_EWORKSPACE
    for field, value, want in (("K", 384, L.MOE_EINVAL), ("lda", 513, L.MOE_EINVAL), ("ldb", 520, L.MOE_EINVAL),
                               ("b_group_stride", 64 * 512 + 1, L.MOE_EINVAL), ("ragged_k", 1, L.MOE_ENOTSUP),
                               ("G", 1024, L.MOE_ENOTSUP), ("a_scale", None, L.MOE_EINVAL),
                               ("b_dtype", L.MOE_E4M3, L.MOE_ENOTSUP)):
        bad = L.MoeGemmArgs.from_buffer_copy(a)
        setattr(bad, field, value)
        assert L._lib.moe_grouped_gemm(ctypes.byref(bad), fake, 1 << 20, None) == want, field
    # MXFP8 row tiles: the same 1023-group limit
    a8 = L.MoeGemmArgs.from_buffer_copy(a)
    a8.a_dtype = a8.b_dtype = L.MOE_E4M3
    a8.lda, a8.ldb, a8.b_group_stride = 512, 512, 64 * 512
    a8.G = 1024
    assert L._lib.moe_grouped_gemm(ctypes.byref(a8), fake, 1 << 20, None) == L.MOE_ENOTSUP


def test_host_argument_errors_fused_quant(lib):
    """The GEMM's fused output quantisation: every rejected combination returns its status
    before anything is enqueued; C may be omitted only when a quantised copy is asked for."""
    from dropless_mixture_experts_device_amd import _lib as L
    fake = ctypes.c_void_p(1 << 20)
    M, N, K, G = 128, 64, 512, 4
    cap = L.quant_col_blocks(M, G)
    a = L.MoeGemmArgs(G=G, offsets=fake.value, M=M, N=N, K=K, A=fake.value, a_dtype=L.MOE_E4M3, lda=K, A_rows=M,
                      a_rows=None, B=fake.value, b_dtype=L.MOE_E4M3, ldb=K, b_group_stride=2 * N * K, C=fake.value,
                      c_dtype=L.MOE_BF16, ldc=N, epilogue=L.MOE_EPI_SWIGLU, aux=None, ld_aux=0, a_scale=fake.value,
                      lda_scale=K // 32, b_scale=fake.value, ldb_scale=K // 32, b_scale_group_stride=2 * N * K // 32,
                      ragged_k=0, c_group_stride=0, q_dtype=L.MOE_E4M3, q_row=fake.value, ld_q_row=N,
                      s_row=fake.value, ld_s_row=N // 32, q_col=fake.value, s_col=fake.value,
                      q_block_start=fake.value, q_col_blocks=cap)
    assert L._lib.moe_grouped_gemm(ctypes.byref(a), None, 0, None) == L.MOE_EWORKSPACE
    cases = (("q_dtype", 5, L.MOE_ENOTSUP), ("c_dtype", L.MOE_F32, L.MOE_ENOTSUP),
             ("N", 48, L.MOE_EINVAL), ("q_row", None, L.MOE_EINVAL), ("ld_q_row", N - 16, L.MOE_EINVAL),
             ("ld_q_row", N + 8, L.MOE_EINVAL), ("ld_s_row", 1, L.MOE_EINVAL), ("s_row", None, L.MOE_EINVAL),
             ("s_col", None, L.MOE_EINVAL), ("q_block_start", None, L.MOE_EINVAL),
             ("q_col_blocks", cap - 1, L.MOE_EINVAL), ("q_row", fake.value + 8, L.MOE_EINVAL))
    for field, value, want in cases:
        bad = L.MoeGemmArgs.from_buffer_copy(a)
        setattr(bad, field, value)
        if field == "N":
            bad.ldc, bad.ld_q_row = 48, 48
        assert L._lib.moe_grouped_gemm(ctypes.byref(bad), fake, 1 << 20, None) == want, (field, value)
    # bf16 operands, ragged-K mode and E2M1 column-wise copies are not offered
    for fields, want in (({"a_dtype": L.MOE_BF16, "b_dtype": L.MOE_BF16}, L.MOE_ENOTSUP),
                         ({"q_dtype": L.MOE_E2M1}, L.MOE_ENOTSUP)):
        bad = L.MoeGemmArgs.from_buffer_copy(a)
        for k_, v in fields.items():
            setattr(bad, k_, v)
        assert L._lib.moe_grouped_gemm(ctypes.byref(bad), fake, 1 << 20, None) == want, fields
    bad = L.MoeGemmArgs.from_buffer_copy(a)
    bad.ragged_k, bad.epilogue, bad.b_group_stride, bad.b_scale_group_stride = 1, L.MOE_EPI_NONE, 0, 0
    bad.c_group_stride = M * N
    assert L._lib.moe_grouped_gemm(ctypes.byref(bad), fake, 1 << 20, None) == L.MOE_ENOTSUP
    # quantised outputs given without q_dtype, and a missing C without them, are errors
    bad = L.MoeGemmArgs.from_buffer_copy(a)
    bad.q_dtype = 0
    assert L._lib.moe_grouped_gemm(ctypes.byref(bad), fake, 1 << 20, None) == L.MOE_EINVAL
    plain = L.MoeGemmArgs.from_buffer_copy(a)
    for f_ in ("q_row", "s_row", "q_col", "s_col", "q_block_start"):
        setattr(plain, f_, None)
    plain.q_dtype, plain.C = 0, None
    assert L._lib.moe_grouped_gemm(ctypes.byref(plain), fake, 1 << 20, None) == L.MOE_EINVAL
    # C omitted with a quantised copy requested passes the argument checks (stops at the workspace)
    ok = L.MoeGemmArgs.from_buffer_copy(a)
    ok.C = None
    assert L._lib.moe_grouped_gemm(ctypes.byref(ok), None, 0, None) == L.MOE_EWORKSPACE


def test_binding_constants_match_header_enums():
    """Every enumerator of include/moe.h has the same value in the Python binding, and every
    workspace op id is answered (an unknown one returns 0)."""
    from dropless_mixture_experts_device_amd import _lib as L
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    found = dict((n, int(v)) for n, v in re.findall(r"\b(MOE_[A-Z0-9_]+)\s*=\s*(\d+)", src))
    assert {"MOE_OK", "MOE_BF16", "MOE_SIGMOID", "MOE_OP_ROUTE_BWD", "MOE_OP_COMBINE_BWD_QUANT"} <= set(found)
    for name, value in found.items():
        assert getattr(L, name) == value, name
    ops = [v for n, v in found.items() if n.startswith("MOE_OP_")]
    assert sorted(ops) == list(range(len(ops)))
    assert L.moe_workspace_bytes(max(ops) + 1, 1024, 512, 64, 8, 65) == 0
    assert L.moe_workspace_bytes(found["MOE_OP_ROUTE_BWD"], 1024, 512, 64, 8, 0) > 0
    assert L.moe_workspace_bytes(found["MOE_OP_COMBINE_BWD_QUANT"], 1024, 0, 0, 8, 65) > 1024 * 9 * 4
