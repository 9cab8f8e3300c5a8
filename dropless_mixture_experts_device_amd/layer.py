"""One dropless MoE layer forward on one GPU, composed from the C entry points.

[Reading] "Method overview": route -> dispatch -> compute -> combine.
[Blog] Figure 3 paragraph: the router assigns experts, dispatch moves the tokens, the grouped
MLP runs two grouped GEMMs over the variable-length groups, combine restores token order.

This module only allocates device buffers (through torch) and calls the HIP library in
order; no arithmetic of the layer happens in Python.
"""
from __future__ import annotations

import dataclasses

import torch

from . import _lib as L


@dataclasses.dataclass
class LayerShape:
    T: int
    d: int
    f: int
    E: int
    k: int
    shared: bool = False
    score: int = L.MOE_SOFTMAX
    dtype: torch.dtype = torch.bfloat16

    @property
    def groups(self) -> int:
        return self.E + (1 if self.shared else 0)

    @property
    def rows(self) -> int:
        return self.T * self.k + (self.T if self.shared else 0)


class LayerBuffers:
    """Every intermediate of the forward, allocated once (the layer never allocates while it
    runs, so a forward can be captured in a HIP graph)."""

    def __init__(self, s: LayerShape, device, fused_gather: bool = True, save_gu: bool = False):
        self.shape = s
        self.fused_gather = fused_gather
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.topk_idx = torch.empty((s.T, s.k), **i32)
        self.topk_w = torch.empty((s.T, s.k), dtype=torch.float32, device=dev)
        self.offsets = torch.empty((s.groups + 1,), **i32)
        self.row_of = torch.empty((s.T, s.k), **i32)
        self.src_token = torch.empty((s.rows,), **i32)
        self.x_perm = None if fused_gather else torch.empty((s.rows, s.d), dtype=s.dtype, device=dev)
        self.H = torch.empty((s.rows, s.f), dtype=s.dtype, device=dev)
        self.GU = torch.empty((s.rows, 2 * s.f), dtype=s.dtype, device=dev) if save_gu else None
        self.Y = torch.empty((s.rows, s.d), dtype=s.dtype, device=dev)
        self.out = torch.empty((s.T, s.d), dtype=s.dtype, device=dev)
        pb = L.moe_workspace_bytes(L.MOE_OP_PERMUTE, s.T, s.d, s.E, s.k, 0)
        gb = L.moe_workspace_bytes(L.MOE_OP_GROUPED_GEMM, 0, 0, 0, 0, s.groups)
        rb = L.moe_workspace_bytes(L.MOE_OP_ROUTE, s.T, s.d, s.E, s.k, 0)
        self.ws_route = torch.empty((max(rb, 256),), dtype=torch.uint8, device=dev)
        self.ws_permute = torch.empty((max(pb, 256),), dtype=torch.uint8, device=dev)
        self.ws_gemm1 = torch.empty((max(gb, 256),), dtype=torch.uint8, device=dev)
        self.ws_gemm2 = torch.empty((max(gb, 256),), dtype=torch.uint8, device=dev)


def route(x, w_router, bias, s: LayerShape, b: LayerBuffers, keys_out=None):
    L.moe_route(x, w_router, bias, s.k, s.score, b.topk_idx, b.topk_w, keys_out, workspace=b.ws_route)


def permute(x, s: LayerShape, b: LayerBuffers):
    L.moe_permute(None if b.fused_gather else x, b.topk_idx, s.E, s.shared, b.offsets, b.row_of, b.src_token,
                  b.x_perm, b.ws_permute, d=s.d, dtype=L._dtype(x))


def experts(x, w_gu, w_down, s: LayerShape, b: LayerBuffers):
    if b.fused_gather:
        L.moe_grouped_gemm(x, w_gu, b.H, b.offsets, L.MOE_EPI_SWIGLU, a_rows=b.src_token, aux=b.GU,
                           workspace=b.ws_gemm1)
    else:
        L.moe_grouped_gemm(b.x_perm, w_gu, b.H, b.offsets, L.MOE_EPI_SWIGLU, aux=b.GU, workspace=b.ws_gemm1)
    L.moe_grouped_gemm(b.H, w_down, b.Y, b.offsets, L.MOE_EPI_NONE, workspace=b.ws_gemm2)


def combine(s: LayerShape, b: LayerBuffers):
    tk = s.T * s.k
    L.moe_combine(b.Y[:tk], b.topk_w, b.row_of, b.Y[tk:] if s.shared else None, b.out)


def forward(x, w_router, bias, w_gu, w_down, s: LayerShape, b: LayerBuffers):
    """out = combine(experts(permute(x, route(x)))); w_gu [E(+1), 2f, d] (gate rows first),
    w_down [E(+1), d, f]; slot E holds the shared expert when s.shared. Returns b.out."""
    route(x, w_router, bias, s, b)
    permute(x, s, b)
    experts(x, w_gu, w_down, s, b)
    combine(s, b)
    return b.out


# --------------------------------------------------------------------------------------
# MXFP8 training step (forward + backward of the experts, the permutation and the combine)
#
# [Blog] "Optimisations dropless MoE needs": the expert GEMMs run in MXFP8 with group-aware
# quantisation; [Reading] contribution 3: MoE low precision needs group quantisation.
# Every GEMM operand is quantised along that GEMM's contraction axis: row-wise for the
# forward and data-gradient GEMMs, in 32-row blocks inside each group (column-wise, output
# transposed) for the weight gradients, whose contraction runs over the group's tokens.
# --------------------------------------------------------------------------------------

def _u8(shape, dev):
    return torch.empty(shape, dtype=torch.uint8, device=dev)


class MxWeights:
    """The step's quantised weights, both axis copies (quantised once per step):
    gu / dn     row-wise along d (W_gu [G, 2f, d]) and along f (W_down [G, d, f]) for the forward;
    guT / dnT   along 2f and along d (column-wise over the stacked weights, transposed) for
                the data gradients, viewed per group as [G, d, 2f] and [G, f, d]."""

    def __init__(self, s: LayerShape, device):
        dev = torch.device(device)
        G, d, f = s.groups, s.d, s.f
        for n, k in (("d", d), ("f", f), ("2f", 2 * f)):
            if k % 128:
                raise ValueError(f"MXFP8 GEMMs need {n} % 128 == 0 (got {k})")
        self.shape = s
        self.q_gu, self.s_gu = _u8((G, 2 * f, d), dev), _u8((G, 2 * f, d // 32), dev)
        self.q_dn, self.s_dn = _u8((G, d, f), dev), _u8((G, d, f // 32), dev)
        cgu = L.quant_col_blocks(G * 2 * f, G)
        cdn = L.quant_col_blocks(G * d, G)
        self.q_guT, self.s_guT = _u8((d, 32 * cgu), dev), _u8((d, cgu), dev)
        self.q_dnT, self.s_dnT = _u8((f, 32 * cdn), dev), _u8((f, cdn), dev)
        self.off_gu = (torch.arange(G + 1, dtype=torch.int32, device=dev) * (2 * f)).contiguous()
        self.off_dn = (torch.arange(G + 1, dtype=torch.int32, device=dev) * d).contiguous()
        self.bs = torch.empty((G + 1,), dtype=torch.int32, device=dev)

    def quantise(self, w_gu, w_down):
        """Both copies of each weight stack from one read of it (2f and d are multiples of 128,
        so group g's transposed blocks start at g*2f/32 and g*d/32)."""
        s = self.shape
        G, d, f = s.groups, s.d, s.f
        L.moe_group_quant_mxfp8_dual(w_gu.view(G * 2 * f, d), self.q_gu.view(G * 2 * f, d),
                                     self.s_gu.view(G * 2 * f, d // 32), self.q_guT, self.s_guT, self.off_gu,
                                     block_start=self.bs)
        L.moe_group_quant_mxfp8_dual(w_down.view(G * d, f), self.q_dn.view(G * d, f), self.s_dn.view(G * d, f // 32),
                                     self.q_dnT, self.s_dnT, self.off_dn, block_start=self.bs)

    # The column-wise quantiser writes each group's transposed block contiguously (group-major);
    # with 2f and d multiples of 128 there is no padding, so the copies are plain [G, ., .] arrays.
    def gu_T(self):
        s = self.shape
        G, d, f2 = s.groups, s.d, 2 * s.f
        return (self.q_guT.view(-1)[:G * d * f2].view(G, d, f2),
                self.s_guT.view(-1)[:G * d * f2 // 32].view(G, d, f2 // 32))

    def dn_T(self):
        s = self.shape
        G, d, f = s.groups, s.d, s.f
        return (self.q_dnT.view(-1)[:G * f * d].view(G, f, d),
                self.s_dnT.view(-1)[:G * f * d // 32].view(G, f, d // 32))


class MxBuffers(LayerBuffers):
    """Everything the MXFP8 forward and backward write, allocated once."""

    def __init__(self, s: LayerShape, device):
        super().__init__(s, device, fused_gather=True, save_gu=True)
        dev = torch.device(device)
        R, G, d, f = s.rows, s.groups, s.d, s.f
        cap = L.quant_col_blocks(R, G)
        bf = dict(dtype=torch.bfloat16, device=dev)
        self.q_x, self.s_x = _u8((s.T, d), dev), _u8((s.T, d // 32), dev)
        self.q_h, self.s_h = _u8((R, f), dev), _u8((R, f // 32), dev)
        # backward
        self.dY = torch.empty((R, d), **bf)
        self.dw = torch.empty((s.T, s.k), dtype=torch.float32, device=dev)
        self.q_dy, self.s_dy = _u8((R, d), dev), _u8((R, d // 32), dev)
        self.dH = torch.empty((R, f), **bf)
        self.dGU = torch.empty((R, 2 * f), **bf)
        self.q_dgu, self.s_dgu = _u8((R, 2 * f), dev), _u8((R, 2 * f // 32), dev)
        self.dXp = torch.empty((R, d), **bf)
        self.dx = torch.empty((s.T, d), **bf)
        # column-wise (weight-gradient) operands, transposed, groups on 128-row boundaries
        self.qc_dy, self.sc_dy = _u8((d, 32 * cap), dev), _u8((d, cap), dev)
        self.qc_h, self.sc_h = _u8((f, 32 * cap), dev), _u8((f, cap), dev)
        self.qc_dgu, self.sc_dgu = _u8((2 * f, 32 * cap), dev), _u8((2 * f, cap), dev)
        self.qc_x, self.sc_x = _u8((d, 32 * cap), dev), _u8((d, cap), dev)
        self.bs = torch.empty((G + 1,), dtype=torch.int32, device=dev)
        self.dW_gu = torch.empty((G, 2 * f, d), **bf)
        self.dW_down = torch.empty((G, d, f), **bf)
        # the router's backward: keys saved by the forward, fp32 gradients of its parameters
        self.keys = torch.empty((s.T, s.E), dtype=torch.float32, device=dev)
        self.dW_router = torch.empty((s.E, d), dtype=torch.float32, device=dev)
        self.d_bias = torch.empty((s.E,), dtype=torch.float32, device=dev)
        rbb = L.moe_workspace_bytes(L.MOE_OP_ROUTE_BWD, s.T, d, s.E, s.k, 0)
        self.ws_route_bwd = torch.empty((rbb,), dtype=torch.uint8, device=dev)
        cqb = L.moe_workspace_bytes(L.MOE_OP_COMBINE_BWD_QUANT, s.T, 0, 0, s.k, G)
        self.ws_combine_quant = torch.empty((cqb,), dtype=torch.uint8, device=dev)
        gb = L.moe_workspace_bytes(L.MOE_OP_GROUPED_GEMM, 0, 0, 0, 0, G)
        self.ws_gemm3 = torch.empty((max(gb, 256),), dtype=torch.uint8, device=dev)


def _nomark(name):
    pass


def forward_mx(x, w_router, bias, mw: MxWeights, s: LayerShape, b: MxBuffers, routed: bool = False, mark=None,
               fuse_h_quant: bool = True, write_h: bool = True):
    """MXFP8 forward: route and permute as in bf16, x quantised row-wise once per token (the
    GEMM gathers codes and scale rows through src_token), GEMM 1 + SwiGLU saving G and U,
    H quantised row-wise (and column-wise for the backward's wgrad 2), GEMM 2, combine.
    mw must hold this step's quantised weights.
    fuse_h_quant (the default): GEMM 1's epilogue writes both quantised copies of H (the same
    bytes as the standalone dual pass over the stored H, which fuse_h_quant=False runs);
    write_h=False then leaves the bf16 H unwritten (the step reads only its quantised copies).
    routed=True skips the router: b.topk_idx and b.topk_w already hold the assignment.
    Otherwise the router's keys are kept in b.keys for its backward.
    mark(name), if given, is called after each stage (e.g. to record a timing event)."""
    mark = mark or _nomark
    if not routed:
        route(x, w_router, bias, s, b, keys_out=b.keys)
    mark("route")
    permute(x, s, b)
    mark("permute")
    L.moe_group_quant_mxfp8(x, b.q_x, b.s_x, axis=0)
    mark("quant_x")
    if fuse_h_quant:
        L.moe_grouped_gemm(b.q_x, mw.q_gu, b.H if write_h else None, b.offsets, L.MOE_EPI_SWIGLU, a_rows=b.src_token,
                           aux=b.GU, workspace=b.ws_gemm1, a_scale=b.s_x, b_scale=mw.s_gu, q_row=b.q_h, s_row=b.s_h,
                           q_col=b.qc_h, s_col=b.sc_h, q_block_start=b.bs, out_shape=(s.rows, s.f))
        mark("gemm1_swiglu")
    else:
        L.moe_grouped_gemm(b.q_x, mw.q_gu, b.H, b.offsets, L.MOE_EPI_SWIGLU, a_rows=b.src_token, aux=b.GU,
                           workspace=b.ws_gemm1, a_scale=b.s_x, b_scale=mw.s_gu)
        mark("gemm1_swiglu")
        L.moe_group_quant_mxfp8_dual(b.H, b.q_h, b.s_h, b.qc_h, b.sc_h, b.offsets, block_start=b.bs)
        mark("quant_h")
    L.moe_grouped_gemm(b.q_h, mw.q_dn, b.Y, b.offsets, L.MOE_EPI_NONE, workspace=b.ws_gemm2, a_scale=b.s_h,
                       b_scale=mw.s_dn)
    mark("gemm2")
    combine(s, b)
    mark("combine")
    return b.out


def backward_mx(x, d_out, mw: MxWeights, s: LayerShape, b: MxBuffers, mark=None, w_router=None,
                fuse_swiglu_quant: bool = True, fuse_combine_quant: bool = True, swiglu_in_dgrad2: bool = True):
    """Backward of forward_mx given d_out [T, d]: fills b.dx, b.dw, b.dW_gu, b.dW_down and,
    when w_router is given (a forward that ran the router), b.dW_router and b.d_bias.

    combine^T -> dY; dgrad 2 (dH = dY W_down, contracted over d) and wgrad 2 (dW_down[g] =
    dY_g^T H_g over the group's tokens); SwiGLU backward from the saved G, U; dgrad 1
    (dX_perm = dGU W_gu, over 2f) and wgrad 1 (dW_gu[g] = dGU_g^T X_g); permute^T -> dx;
    then the router's backward: the routing weights' gradient dw through the top-k
    normalisation to the keys, from there to W_router and the bias, and the router's share
    of the input gradient added into dx (its dx pass forms permute^T itself). With fuse_swiglu_quant (the default) the SwiGLU
    backward is not written out: with swiglu_in_dgrad2 (the default) dgrad 2's epilogue forms
    dGU from its dH tile and the saved G, U and writes both MXFP8 copies of dGU (b.dH and b.dGU
    are not written), else the quantiser that writes those copies forms dGU from the stored
    dH; without fuse_swiglu_quant dGU is written by its own kernel and then quantised. Likewise with
    fuse_combine_quant (the default) dY is formed inside the quantiser from d_out and the
    routing weights, so b.dY is not written and the combine's transpose only computes dw."""
    mark = mark or _nomark
    tk = s.T * s.k
    if fuse_combine_quant:
        L.moe_combine_backward(d_out, b.topk_w, b.row_of, None, y=b.Y[:tk], dw=b.dw)
        mark("combine_bwd")
        L.moe_combine_backward_quant_mxfp8_dual(d_out, b.topk_w, b.row_of, b.src_token, s.shared, b.q_dy, b.s_dy,
                                                b.qc_dy, b.sc_dy, b.offsets, block_start=b.bs,
                                                workspace=b.ws_combine_quant)
        mark("quant_dy")
    else:
        L.moe_combine_backward(d_out, b.topk_w, b.row_of, b.dY[:tk], y=b.Y[:tk],
                               dy_shared=b.dY[tk:] if s.shared else None, dw=b.dw)
        mark("combine_bwd")
        L.moe_group_quant_mxfp8_dual(b.dY, b.q_dy, b.s_dy, b.qc_dy, b.sc_dy, b.offsets, block_start=b.bs)
        mark("quant_dy")
    # dgrad 2 and wgrad 2
    q_dnT, s_dnT = mw.dn_T()
    in_dgrad2 = fuse_swiglu_quant and swiglu_in_dgrad2
    if in_dgrad2:
        L.moe_grouped_gemm(b.q_dy, q_dnT, None, b.offsets, L.MOE_EPI_SWIGLU_BWD, aux=b.GU, workspace=b.ws_gemm1,
                           a_scale=b.s_dy, b_scale=s_dnT, q_row=b.q_dgu, s_row=b.s_dgu, q_col=b.qc_dgu, s_col=b.sc_dgu,
                           q_block_start=b.bs, out_shape=(s.rows, 2 * s.f))
    else:
        L.moe_grouped_gemm(b.q_dy, q_dnT, b.dH, b.offsets, L.MOE_EPI_NONE, workspace=b.ws_gemm1, a_scale=b.s_dy,
                           b_scale=s_dnT)
    mark("dgrad2")
    L.moe_grouped_gemm(b.qc_dy, b.qc_h, b.dW_down, b.bs, L.MOE_EPI_NONE, workspace=b.ws_gemm3,
                       a_scale=b.sc_dy, b_scale=b.sc_h, ragged_k=True)
    mark("wgrad2")
    # SwiGLU backward, dgrad 1 and wgrad 1
    if in_dgrad2:
        pass
    elif fuse_swiglu_quant:
        L.moe_swiglu_backward_quant_mxfp8_dual(b.dH, b.GU, b.q_dgu, b.s_dgu, b.qc_dgu, b.sc_dgu, b.offsets,
                                               block_start=b.bs)
        mark("swiglu_bwd_quant_dgu")
    else:
        L.moe_swiglu_backward(b.dH, b.GU, b.dGU)
        mark("swiglu_bwd")
        L.moe_group_quant_mxfp8_dual(b.dGU, b.q_dgu, b.s_dgu, b.qc_dgu, b.sc_dgu, b.offsets, block_start=b.bs)
        mark("quant_dgu")
    q_guT, s_guT = mw.gu_T()
    L.moe_grouped_gemm(b.q_dgu, q_guT, b.dXp, b.offsets, L.MOE_EPI_NONE, workspace=b.ws_gemm2, a_scale=b.s_dgu,
                       b_scale=s_guT)
    mark("dgrad1")
    L.moe_group_quant_mxfp8(x, b.qc_x, b.sc_x, axis=1, group_offsets=b.offsets, block_start=b.bs,
                            row_index=b.src_token)
    mark("quant_cols_x")
    L.moe_grouped_gemm(b.qc_dgu, b.qc_x, b.dW_gu, b.bs, L.MOE_EPI_NONE, workspace=b.ws_gemm3,
                       a_scale=b.sc_dgu, b_scale=b.sc_x, ragged_k=True)
    mark("wgrad1")
    if w_router is None:
        # permute^T: each token's rows summed back (plus the shared expert's row)
        L.moe_combine(b.dXp[:tk], None, b.row_of, b.dXp[tk:] if s.shared else None, b.dx)
        mark("unpermute")
    else:
        # the router's backward; its dx pass forms permute^T itself (the same sum and rounding
        # as moe_combine without weights) and adds the router's share
        L.moe_route_backward(x, w_router, b.keys, b.topk_idx, b.dw, s.score, b.row_of, offsets=b.offsets,
                             src_token=b.src_token, d_x=b.dx, d_x_perm=b.dXp[:tk],
                             d_x_perm_shared=b.dXp[tk:] if s.shared else None, d_w_router=b.dW_router,
                             d_bias=b.d_bias, workspace=b.ws_route_bwd)
        mark("unpermute_route_bwd")


# --------------------------------------------------------------------------------------
# MXFP4 forward ([Blog] "JAX plus Transformer Engine MoE training performance": a 4-bit
# block-scaled format is the planned next precision; [Reading] contribution 3: FP8/FP4
# recipes). Every GEMM operand is quantised row-wise along its contraction axis, as in the
# MXFP8 forward, to E2M1 codes packed two per byte with an E8M0 scale per 32 elements.
# --------------------------------------------------------------------------------------

class Mx4Weights:
    """Row-wise MXFP4 copies of the expert weights: W_gu [G, 2f, d] along d and W_down
    [G, d, f] along f (codes [., ., K/2] bytes, scales [., ., K/32])."""

    def __init__(self, s: LayerShape, device):
        dev = torch.device(device)
        G, d, f = s.groups, s.d, s.f
        for n, k in (("d", d), ("f", f)):
            if k % 256:
                raise ValueError(f"MXFP4 GEMMs need {n} % 256 == 0 (got {k})")
        self.shape = s
        self.q_gu, self.s_gu = _u8((G, 2 * f, d // 2), dev), _u8((G, 2 * f, d // 32), dev)
        self.q_dn, self.s_dn = _u8((G, d, f // 2), dev), _u8((G, d, f // 32), dev)

    def quantise(self, w_gu, w_down):
        s = self.shape
        G, d, f = s.groups, s.d, s.f
        L.moe_group_quant_mxfp4(w_gu.view(G * 2 * f, d), self.q_gu.view(G * 2 * f, d // 2),
                                self.s_gu.view(G * 2 * f, d // 32))
        L.moe_group_quant_mxfp4(w_down.view(G * d, f), self.q_dn.view(G * d, f // 2), self.s_dn.view(G * d, f // 32))


class Mx4Buffers(LayerBuffers):
    """The MXFP4 forward's intermediates: the bf16 ones of the layer plus the quantised x and H."""

    def __init__(self, s: LayerShape, device):
        super().__init__(s, device, fused_gather=True)
        dev = torch.device(device)
        self.q_x, self.s_x = _u8((s.T, s.d // 2), dev), _u8((s.T, s.d // 32), dev)
        self.q_h, self.s_h = _u8((s.rows, s.f // 2), dev), _u8((s.rows, s.f // 32), dev)


def forward_mx4(x, w_router, bias, mw: Mx4Weights, s: LayerShape, b: Mx4Buffers, routed: bool = False, mark=None,
                fuse_h_quant: bool = True, write_h: bool = True):
    """MXFP4 forward: route and permute as in bf16, x quantised once per token (GEMM 1 gathers
    its code and scale rows through src_token), GEMM 1 + SwiGLU with H quantised in its
    epilogue (fuse_h_quant=False: bf16 H, then a separate quantiser pass; write_h=False: the
    bf16 H is not written), GEMM 2, combine. mw must hold the quantised weights; routed=True
    keeps b.topk_idx and b.topk_w as they are; mark(name), if given, is called after each stage."""
    mark = mark or _nomark
    if not routed:
        route(x, w_router, bias, s, b)
    mark("route")
    permute(x, s, b)
    mark("permute")
    L.moe_group_quant_mxfp4(x, b.q_x, b.s_x)
    mark("quant_x")
    if fuse_h_quant:
        L.moe_grouped_gemm(b.q_x, mw.q_gu, b.H if write_h else None, b.offsets, L.MOE_EPI_SWIGLU, a_rows=b.src_token,
                           workspace=b.ws_gemm1, a_scale=b.s_x, b_scale=mw.s_gu, fp4=True, q_row=b.q_h, s_row=b.s_h,
                           q_fp4=True, out_shape=(s.rows, s.f))
        mark("gemm1_swiglu")
    else:
        L.moe_grouped_gemm(b.q_x, mw.q_gu, b.H, b.offsets, L.MOE_EPI_SWIGLU, a_rows=b.src_token,
                           workspace=b.ws_gemm1, a_scale=b.s_x, b_scale=mw.s_gu, fp4=True)
        mark("gemm1_swiglu")
        L.moe_group_quant_mxfp4(b.H, b.q_h, b.s_h)
        mark("quant_h")
    L.moe_grouped_gemm(b.q_h, mw.q_dn, b.Y, b.offsets, L.MOE_EPI_NONE, workspace=b.ws_gemm2, a_scale=b.s_h,
                       b_scale=mw.s_dn, fp4=True)
    mark("gemm2")
    combine(s, b)
    mark("combine")
    return b.out
