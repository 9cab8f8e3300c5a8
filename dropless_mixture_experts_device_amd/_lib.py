"""ctypes binding of libmoe.so: one Python function per C entry point, same names.

Only argument marshalling lives here (tensor -> device pointer, the current HIP stream,
status -> exception). Every step of the computation runs in the HIP library; there is no
fallback: if libmoe.so is missing or fails to load, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

# MOE_LIB selects another build of the same library (the debug or host-ASan variants)
_LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; run dropless_mixture_experts_device_amd.build.build()")
_lib = ctypes.CDLL(_LIB_PATH)

MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_EWORKSPACE, MOE_EHIP = 0, 1, 2, 3, 4
MOE_F32, MOE_BF16, MOE_E4M3, MOE_E2M1 = 0, 1, 2, 3
MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_EPI_NONE, MOE_EPI_SWIGLU, MOE_EPI_SWIGLU_BWD = 0, 1, 2
MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_GROUPED_GEMM, MOE_OP_QUANT, MOE_OP_ROUTE_BWD, MOE_OP_COMBINE_BWD_QUANT = 0, 1, 2, 3, 4, 5

_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


class MoeGemmArgs(ctypes.Structure):
    """Mirror of moe_gemm_args_t (include/moe.h)."""
    _fields_ = [
        ("G", _i32), ("offsets", _vp), ("M", _i64), ("N", _i64), ("K", _i64),
        ("A", _vp), ("a_dtype", _i32), ("lda", _i64), ("A_rows", _i64), ("a_rows", _vp),
        ("B", _vp), ("b_dtype", _i32), ("ldb", _i64), ("b_group_stride", _i64),
        ("C", _vp), ("c_dtype", _i32), ("ldc", _i64),
        ("epilogue", _i32), ("aux", _vp), ("ld_aux", _i64),
        ("a_scale", _vp), ("lda_scale", _i64), ("b_scale", _vp), ("ldb_scale", _i64), ("b_scale_group_stride", _i64),
        ("ragged_k", _i32), ("c_group_stride", _i64),
        ("q_dtype", _i32), ("q_row", _vp), ("ld_q_row", _i64), ("s_row", _vp), ("ld_s_row", _i64),
        ("q_col", _vp), ("s_col", _vp), ("q_block_start", _vp), ("q_col_blocks", _i64),
    ]


_lib.moe_status_str.argtypes = [_i32]
_lib.moe_status_str.restype = ctypes.c_char_p
_lib.moe_workspace_bytes.argtypes = [_i32, _i64, _i64, _i32, _i32, _i32]
_lib.moe_workspace_bytes.restype = _sz
_lib.moe_route.argtypes = [_vp, _vp, _i32, _vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moe_route.restype = _i32
_lib.moe_permute.argtypes = [_vp, _i32, _vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moe_permute.restype = _i32
_lib.moe_grouped_gemm.argtypes = [ctypes.POINTER(MoeGemmArgs), _vp, _sz, _vp]
_lib.moe_grouped_gemm.restype = _i32
_lib.moe_combine.argtypes = [_vp, _i32, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp]
_lib.moe_combine.restype = _i32
_lib.moe_group_quant_mxfp8.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i32, _i32, _vp, _i64, _vp, _i64,
                                       _vp, _vp, _sz, _vp]
_lib.moe_group_quant_mxfp8.restype = _i32
_lib.moe_group_quant_mxfp4.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]
_lib.moe_group_quant_mxfp4.restype = _i32
_lib.moe_group_quant_mxfp8_dual.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i32, _vp, _i64, _vp, _i64,
                                            _vp, _i64, _vp, _i64, _vp, _vp, _sz, _vp]
_lib.moe_group_quant_mxfp8_dual.restype = _i32

_lib.moe_combine_backward.argtypes = [_vp, _i32, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp, _vp, _vp]
_lib.moe_combine_backward.restype = _i32
_lib.moe_swiglu_backward.argtypes = [_vp, _i64, _vp, _i64, _i32, _i64, _i64, _vp, _i64, _vp]
_lib.moe_swiglu_backward.restype = _i32
_lib.moe_route_backward.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp,
                                    _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moe_route_backward.restype = _i32
_lib.moe_swiglu_backward_quant_mxfp8_dual.argtypes = [_vp, _i64, _vp, _i64, _i32, _i64, _i64, _vp, _i32, _vp, _i64,
                                                      _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _sz, _vp]
_lib.moe_swiglu_backward_quant_mxfp8_dual.restype = _i32
_lib.moe_combine_backward_quant_mxfp8_dual.argtypes = [_vp, _i32, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _vp, _i32,
                                                       _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _sz, _vp]
_lib.moe_combine_backward_quant_mxfp8_dual.restype = _i32

EXPORTED = ("moe_status_str", "moe_workspace_bytes", "moe_route", "moe_permute", "moe_grouped_gemm", "moe_combine",
            "moe_group_quant_mxfp8", "moe_group_quant_mxfp8_dual", "moe_group_quant_mxfp4", "moe_combine_backward", "moe_swiglu_backward",
            "moe_route_backward", "moe_swiglu_backward_quant_mxfp8_dual", "moe_combine_backward_quant_mxfp8_dual")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {moe_status_str(status)}")
        self.status = status


def moe_status_str(status: int) -> str:
    return _lib.moe_status_str(status).decode()


def moe_workspace_bytes(op: int, T: int = 0, d: int = 0, E: int = 0, k: int = 0, G: int = 0) -> int:
    return int(_lib.moe_workspace_bytes(op, T, d, E, k, G))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype(t) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.uint8:
        return MOE_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _ws(ws):
    return (_ptr(ws), 0 if ws is None else ws.numel() * ws.element_size())


def moe_route(x, w_router, bias, k: int, score: int, topk_idx, topk_w, keys_out=None, workspace=None, stream=None):
    """x [T,d], w_router [E,d] (bf16 or fp32), bias [E] fp32 or None -> topk_idx int32 [T,k],
    topk_w fp32 [T,k], keys_out fp32 [T,E] (optional). `workspace`: a uint8 device tensor of
    moe_workspace_bytes(MOE_OP_ROUTE, T, d, E) bytes (None when that is zero)."""
    T, d = x.shape
    E = w_router.shape[0]
    ws, wsb = _ws(workspace)
    _check("moe_route", _lib.moe_route(_ptr(x), _ptr(w_router), _dtype(x), _ptr(bias), T, d, E, k, score,
                                       _ptr(topk_idx), _ptr(topk_w), _ptr(keys_out), ws, wsb, _stream(stream)))


def moe_permute(x, topk_idx, E: int, shared_group: bool, offsets, row_of, src_token, x_perm, workspace,
                stream=None, d: int | None = None, dtype: int | None = None):
    """topk_idx int32 [T,k] -> offsets [E+1(+1)], row_of [T,k], src_token [T*k(+T)], and x_perm
    [T*k(+T), d] = x[src_token] when x_perm is given."""
    T, k = topk_idx.shape
    if d is None:
        d = x.shape[1] if x is not None else 0
    if dtype is None:
        dtype = _dtype(x) if x is not None else MOE_BF16
    ws, wsb = _ws(workspace)
    _check("moe_permute", _lib.moe_permute(_ptr(x), dtype, _ptr(topk_idx), T, d, E, k, 1 if shared_group else 0,
                                           _ptr(offsets), _ptr(row_of), _ptr(src_token), _ptr(x_perm), ws, wsb,
                                           _stream(stream)))


def moe_grouped_gemm(A, B, C, offsets, epilogue: int = MOE_EPI_NONE, a_rows=None, aux=None, workspace=None,
                     stream=None, a_scale=None, b_scale=None, ragged_k: bool = False, fp4: bool = False,
                     q_row=None, s_row=None, q_col=None, s_col=None, q_block_start=None, q_fp4: bool = False,
                     out_shape=None):
    """One launch over all groups.

    Ragged rows (default): C[rows of g] = A[a_rows or rows of g] @ B[g]^T (SWIGLU: silu(gate)
    * up). A [A_rows, K]; B [G, N or 2N, K] (any strides with unit inner stride, e.g. a
    permuted view of transposed weights); C [M, N]; offsets int32 [G+1] (device); a_rows
    int32 [M]. MXFP8: A and B are uint8 E4M3 codes with a_scale [A_rows, K/32] and b_scale
    [G, N_B, K/32] uint8 E8M0 bytes. fp4 (MXFP4): A [A_rows, K/2] and B [G, N_B, K/2] uint8
    hold E2M1 codes two per byte (K counts elements, strides are passed in elements).
    Fused output quantisation: q_row / s_row (uint8) receive the row-wise MXFP8 (q_fp4: MXFP4,
    packed) copy of the bf16 output, q_col / s_col / q_block_start the group-aware column-wise
    MXFP8 copy (as moe_group_quant_mxfp8 axis 1). C may then be None, with out_shape = (M, N).
    ragged_k: C [G, M, N], C[g] = A_g @ B_g^T over group g's offsets[g] .. offsets[g+1]-1
    blocks of 32 K elements, A, B, a_scale, b_scale being the column-wise quantiser's
    group-major output buffers (capacities [M, K], [N, K], [M, K/32], [N, K/32]).
    """
    if ragged_k:
        G, M, N = C.shape
        K = A.shape[1]
        args = MoeGemmArgs(
            G=G, offsets=offsets.data_ptr(), M=M, N=N, K=K,
            A=A.data_ptr(), a_dtype=_dtype(A), lda=A.stride(0), A_rows=A.shape[0], a_rows=None,
            B=B.data_ptr(), b_dtype=_dtype(B), ldb=B.stride(0), b_group_stride=0,
            C=C.data_ptr(), c_dtype=_dtype(C), ldc=C.stride(1), epilogue=epilogue, aux=None, ld_aux=0,
            a_scale=None if a_scale is None else a_scale.data_ptr(),
            lda_scale=0 if a_scale is None else a_scale.stride(0),
            b_scale=None if b_scale is None else b_scale.data_ptr(),
            ldb_scale=0 if b_scale is None else b_scale.stride(0), b_scale_group_stride=0,
            ragged_k=1, c_group_stride=C.stride(0))
    else:
        G = B.shape[0]
        M, N = C.shape if C is not None else out_shape
        if epilogue == MOE_EPI_SWIGLU_BWD:
            N //= 2                          # C holds [dg | du]
        per = 2 if fp4 else 1                # elements per stored byte
        if fp4 and (A.dtype != torch.uint8 or B.dtype != torch.uint8):
            raise TypeError("MXFP4 operands are uint8 tensors of packed E2M1 codes")
        K = A.shape[1] * per
        ab = MOE_E2M1 if fp4 else _dtype(A)
        args = MoeGemmArgs(
            G=G, offsets=offsets.data_ptr(), M=M, N=N, K=K,
            A=A.data_ptr(), a_dtype=ab, lda=A.stride(0) * per, A_rows=A.shape[0],
            a_rows=None if a_rows is None else a_rows.data_ptr(),
            B=B.data_ptr(), b_dtype=MOE_E2M1 if fp4 else _dtype(B), ldb=B.stride(1) * per,
            b_group_stride=B.stride(0) * per,
            C=None if C is None else C.data_ptr(), c_dtype=MOE_BF16 if C is None else _dtype(C),
            ldc=N if C is None else C.stride(0),
            epilogue=epilogue, aux=None if aux is None else aux.data_ptr(),
            ld_aux=0 if aux is None else aux.stride(0),
            a_scale=None if a_scale is None else a_scale.data_ptr(),
            lda_scale=0 if a_scale is None else a_scale.stride(0),
            b_scale=None if b_scale is None else b_scale.data_ptr(),
            ldb_scale=0 if b_scale is None else b_scale.stride(1),
            b_scale_group_stride=0 if b_scale is None else b_scale.stride(0), ragged_k=0, c_group_stride=0,
            q_dtype=0 if q_row is None else (MOE_E2M1 if q_fp4 else MOE_E4M3),
            q_row=None if q_row is None else q_row.data_ptr(), ld_q_row=0 if q_row is None else q_row.stride(0),
            s_row=None if s_row is None else s_row.data_ptr(), ld_s_row=0 if s_row is None else s_row.stride(0),
            q_col=None if q_col is None else q_col.data_ptr(), s_col=None if s_col is None else s_col.data_ptr(),
            q_block_start=None if q_block_start is None else q_block_start.data_ptr(),
            q_col_blocks=0 if s_col is None else s_col.shape[1])
    ws, wsb = _ws(workspace)
    _check("moe_grouped_gemm", _lib.moe_grouped_gemm(ctypes.byref(args), ws, wsb, _stream(stream)))


def moe_combine(y, topk_w, row_of, y_shared, out, stream=None):
    """out[t] = sum_j topk_w[t,j] * y[row_of[t,j]] (+ y_shared[t]); topk_w None: weights one
    (the transpose of the permutation's gather)."""
    T, k = row_of.shape
    d = out.shape[1]
    _check("moe_combine", _lib.moe_combine(_ptr(y), _dtype(out), _ptr(topk_w), _ptr(row_of), _ptr(y_shared), T, d, k,
                                           _ptr(out), _stream(stream)))


def quant_col_blocks(rows: int, G: int) -> int:
    """Capacity in 32-row blocks of the column-wise (axis 1) output: 4 * (ceil(rows/128) + G)."""
    return 4 * (-(-rows // 128) + G)


def moe_combine_backward(d_out, topk_w, row_of, dy, y=None, dy_shared=None, dw=None, stream=None):
    """dy[row_of[t,j]] = topk_w[t,j] * d_out[t]; dy_shared[t] = d_out[t]; dw[t,j] = <d_out[t], y[row_of[t,j]]>."""
    T, k = row_of.shape
    d = d_out.shape[1]
    _check("moe_combine_backward", _lib.moe_combine_backward(
        _ptr(d_out), _dtype(d_out), _ptr(topk_w), _ptr(row_of), _ptr(y), T, d, k, _ptr(dy), _ptr(dy_shared),
        _ptr(dw), _stream(stream)))


def moe_route_backward(x, w_router, keys, topk_idx, d_topk_w, score: int, row_of, offsets=None, src_token=None,
                       d_keys_sel=None, d_x=None, d_w_router=None, d_bias=None, workspace=None, stream=None,
                       accumulate_dx: bool = False, d_x_perm=None, d_x_perm_shared=None):
    """Router backward: d_topk_w [T,k] fp32 -> d_keys_sel [T,k] fp32, d_x [T,d] (dtype of x; with
    accumulate_dx the router's share is added to what d_x holds; with d_x_perm it is added to the
    permutation's transpose of d_x_perm (+ d_x_perm_shared), formed in the same kernel and
    rounded as moe_combine would store it), d_w_router [E,d] fp32,
    d_bias [E] fp32 (each optional). keys [T,E] fp32 and topk_idx come from
    moe_route, offsets / row_of / src_token from moe_permute. `workspace`: a uint8 device tensor of
    moe_workspace_bytes(MOE_OP_ROUTE_BWD, T, d, E, k) bytes."""
    T, d = x.shape
    E = w_router.shape[0]
    k = topk_idx.shape[1]
    ws, wsb = _ws(workspace)
    _check("moe_route_backward", _lib.moe_route_backward(
        _ptr(x), _ptr(w_router), _dtype(x), _ptr(keys), _ptr(topk_idx), _ptr(d_topk_w), _ptr(offsets), _ptr(row_of),
        _ptr(src_token), T, d, E, k, score, _ptr(d_keys_sel), _ptr(d_x), int(accumulate_dx), _ptr(d_x_perm),
        _ptr(d_x_perm_shared), _ptr(d_w_router), _ptr(d_bias), ws, wsb,
        _stream(stream)))


def moe_swiglu_backward_quant_mxfp8_dual(dh, gu, q_row, s_row, q_col, s_col, group_offsets, block_start=None,
                                         workspace=None, stream=None):
    """The SwiGLU backward of (dh [rows, f], gu [rows, 2f]) quantised straight into both MXFP8
    copies (as moe_swiglu_backward followed by moe_group_quant_mxfp8_dual, without the bf16
    gate/up gradient in memory)."""
    rows, f = dh.shape
    ws, wsb = _ws(workspace)
    _check("moe_swiglu_backward_quant_mxfp8_dual", _lib.moe_swiglu_backward_quant_mxfp8_dual(
        _ptr(dh), dh.stride(0), _ptr(gu), gu.stride(0), _dtype(dh), rows, f, _ptr(group_offsets),
        group_offsets.numel() - 1, _ptr(q_row), q_row.stride(0), _ptr(s_row), s_row.stride(0), _ptr(q_col),
        q_col.stride(0), _ptr(s_col), s_col.stride(0), _ptr(block_start), ws, wsb, _stream(stream)))


def moe_combine_backward_quant_mxfp8_dual(d_out, topk_w, row_of, src_token, shared: bool, q_row, s_row, q_col, s_col,
                                          group_offsets, block_start=None, workspace=None, stream=None):
    """The combine's transpose (dY rows = topk_w * d_out in expert order, plus d_out as the
    shared rows) quantised straight into both MXFP8 copies, without dY in memory. `workspace`:
    moe_workspace_bytes(MOE_OP_COMBINE_BWD_QUANT, T, 0, 0, k, G) bytes."""
    T, k = row_of.shape
    d = d_out.shape[1]
    ws, wsb = _ws(workspace)
    _check("moe_combine_backward_quant_mxfp8_dual", _lib.moe_combine_backward_quant_mxfp8_dual(
        _ptr(d_out), _dtype(d_out), _ptr(topk_w), _ptr(row_of), _ptr(src_token), T, d, k, int(bool(shared)),
        _ptr(group_offsets), group_offsets.numel() - 1, _ptr(q_row), q_row.stride(0), _ptr(s_row), s_row.stride(0),
        _ptr(q_col), q_col.stride(0), _ptr(s_col), s_col.stride(0), _ptr(block_start), ws, wsb, _stream(stream)))


def moe_swiglu_backward(dh, gu, dgu, stream=None):
    """dgu = [dh * u * silu'(g), dh * silu(g)] from gu = [g, u] (all row-major, rows x f / 2f)."""
    rows, f = dh.shape
    _check("moe_swiglu_backward", _lib.moe_swiglu_backward(
        _ptr(dh), dh.stride(0), _ptr(gu), gu.stride(0), _dtype(dh), rows, f, _ptr(dgu), dgu.stride(0),
        _stream(stream)))


def moe_group_quant_mxfp8(x, q, scales, axis: int = 0, group_offsets=None, block_start=None, workspace=None,
                          stream=None, row_index=None, rows=None):
    """MXFP8 quantisation of x (bf16 or fp32, [in_rows, cols]) into E4M3 codes q (uint8) and
    E8M0 scale bytes (uint8). Logical row r reads x[row_index[r]] when row_index is given
    (then `rows` defaults to row_index's length), else x[r]. axis 0: q [rows, >=cols],
    scales [rows, >=cols/32]. axis 1 (blocks of 32 rows inside each group of group_offsets,
    each group starting on a multiple of 4 blocks; transposed group-major output, group g's
    [cols, 32 n_g] codes at byte 32*cols*block_start[g] of q): q [cols, 32*nb] and scales
    [cols, nb] buffers with nb >= quant_col_blocks(rows, G), block_start int32 [G+1]
    (optional output)."""
    in_rows, cols = x.shape
    if rows is None:
        rows = in_rows if row_index is None else row_index.numel()
    G = 0 if group_offsets is None else group_offsets.numel() - 1
    ws, wsb = _ws(workspace)
    _check("moe_group_quant_mxfp8", _lib.moe_group_quant_mxfp8(
        _ptr(x), _dtype(x), rows, cols, x.stride(0), _ptr(row_index), in_rows, _ptr(group_offsets), G, axis,
        _ptr(q), q.stride(0), _ptr(scales), scales.stride(0), _ptr(block_start), ws, wsb, _stream(stream)))


def moe_group_quant_mxfp4(x, q, scales, stream=None, row_index=None, rows=None):
    """Row-wise MXFP4 quantisation of x (bf16 or fp32, [in_rows, cols]) into packed E2M1
    codes q (uint8 [rows, >= cols/2], even element in the low nibble) and E8M0 scale bytes
    (uint8 [rows, >= cols/32]). Logical row r reads x[row_index[r]] when row_index is given
    (then `rows` defaults to row_index's length), else x[r]."""
    in_rows, cols = x.shape
    if rows is None:
        rows = in_rows if row_index is None else row_index.numel()
    _check("moe_group_quant_mxfp4", _lib.moe_group_quant_mxfp4(
        _ptr(x), _dtype(x), rows, cols, x.stride(0), _ptr(row_index), in_rows, _ptr(q), q.stride(0),
        _ptr(scales), scales.stride(0), _stream(stream)))


def moe_group_quant_mxfp8_dual(x, q_row, s_row, q_col, s_col, group_offsets, block_start=None, workspace=None,
                               stream=None, row_index=None, rows=None):
    """Both MXFP8 copies from one read of x: the row-wise copy into q_row / s_row (as axis 0 of
    moe_group_quant_mxfp8) and the group-aware column-wise copy into q_col / s_col (as axis 1)."""
    in_rows, cols = x.shape
    if rows is None:
        rows = in_rows if row_index is None else row_index.numel()
    ws, wsb = _ws(workspace)
    _check("moe_group_quant_mxfp8_dual", _lib.moe_group_quant_mxfp8_dual(
        _ptr(x), _dtype(x), rows, cols, x.stride(0), _ptr(row_index), in_rows, _ptr(group_offsets),
        group_offsets.numel() - 1, _ptr(q_row), q_row.stride(0), _ptr(s_row), s_row.stride(0), _ptr(q_col),
        q_col.stride(0), _ptr(s_col), s_col.stride(0), _ptr(block_start), ws, wsb, _stream(stream)))
