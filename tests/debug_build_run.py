"""The workloads both the release library (in the test process) and the MOE_DEBUG build (in
its child process) run, returning raw output bits for a bit-for-bit comparison."""
import numpy as np
import torch

import moe_inputs as mi
from tests.gpu_util import DeviceWorkload, bits


def run_layer():
    from dropless_mixture_experts_device_amd import _lib as L, layer
    w = mi.WORKLOADS["small_sigmoid"]
    dw = DeviceWorkload(w)
    s = layer.LayerShape(T=w.T, d=w.d, f=w.f, E=w.E, k=w.k, shared=bool(w.shared_f), score=L.MOE_SIGMOID)
    b = layer.LayerBuffers(s, "cuda")
    layer.forward(dw.x, dw.w_router, dw.bias, dw.w_gu, dw.w_down, s, b)
    torch.cuda.synchronize()
    return {"layer_out": bits(b.out), "layer_H": bits(b.H), "layer_offsets": b.offsets.cpu().numpy()}


def run_mx_step():
    from dropless_mixture_experts_device_amd import _lib as L, layer
    w = mi.WORKLOADS["small_mxfp8"]
    dw = DeviceWorkload(w)
    s = layer.LayerShape(T=w.T, d=w.d, f=w.f, E=w.E, k=w.k, shared=bool(w.shared_f), score=L.MOE_SIGMOID)
    mw = layer.MxWeights(s, "cuda")
    mw.quantise(dw.w_gu, dw.w_down)
    b = layer.MxBuffers(s, "cuda")
    layer.forward_mx(dw.x, dw.w_router, dw.bias, mw, s, b, write_h=False)
    d_out = mi.randn_torch(w.seed, mi.D_OUT, 0, w.T, w.d, 1.0, "bf16", "cuda")
    layer.backward_mx(dw.x, d_out, mw, s, b, w_router=dw.w_router)
    torch.cuda.synchronize()
    res = {f"mx_{n}": bits(getattr(b, n)) for n in ("out", "dx", "dW_gu", "dW_down", "dW_router", "q_h")}
    # the column-wise copy is written group-major up to the block prefix's end (32 code bytes per
    # column and block); the buffer's capacity past it is never written, so it is not compared
    nblk = int(b.bs[-1].item())
    res["mx_qc_dgu"] = b.qc_dgu.reshape(-1)[: 32 * b.qc_dgu.shape[0] * nblk].cpu().numpy()
    res["mx_bs"] = b.bs.cpu().numpy()
    return res
