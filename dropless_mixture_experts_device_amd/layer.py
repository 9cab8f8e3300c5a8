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
