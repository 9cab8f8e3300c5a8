"""Helpers shared by the GPU parity tests (no arithmetic of the method lives here)."""
from __future__ import annotations

import numpy as np
import torch

import moe_inputs as mi

F64 = np.float64
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}

# tolerance of the floating-point outputs against the storage-mirroring oracle:
# e_i = |y_i - r_i| / max(|r_i|, rms(r));  bf16 gates max <= 2e-2, mean <= 2e-3.
BF16_MAX_REL, BF16_MEAN_REL = 2e-2, 2e-3
# fp32 storage: the only differences are fp32 accumulation order and fp32 expf/silu
F32_MAX_REL, F32_MEAN_REL = 1e-4, 1e-5
# MXFP8 pipelines against the MX-mirroring oracle: an intermediate that lands on the other
# side of an E4M3 rounding boundary moves one element by up to one E4M3 step (1/16 relative)
MX_MAX_REL, MX_MEAN_REL = 6e-2, 6e-3
# A whole MXFP8 step against the fully independent oracle: every bf16 intermediate the GPU
# rounds one ulp differently can flip the E4M3 code of a block maximum by a whole step (up to
# 1/8 relative), which moves single outputs by ~2/sqrt(K) of the output rms; the mean stays
# at the bf16 level. Stage-wise checks (each stage on the GPU's own inputs) use the bf16 gate.
MX_E2E_MAX_REL, MX_E2E_MEAN_REL = 0.25, 2e-3


def rel_err(y, r):
    y = np.asarray(y, F64)
    r = np.asarray(r, F64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    den = np.maximum(np.abs(r), rms if rms > 0 else 1.0)
    e = np.abs(y - r) / den
    return float(e.max()) if e.size else 0.0, float(e.mean()) if e.size else 0.0


def assert_close(y, r, dtype: str, what: str = ""):
    mx, mean = rel_err(y, r)
    lim = {"bf16": (BF16_MAX_REL, BF16_MEAN_REL), "mx": (MX_MAX_REL, MX_MEAN_REL),
           "mx_e2e": (MX_E2E_MAX_REL, MX_E2E_MEAN_REL)}.get(dtype, (F32_MAX_REL, F32_MEAN_REL))
    assert mx <= lim[0] and mean <= lim[1], f"{what}: max rel {mx:.3e} mean rel {mean:.3e} (limits {lim})"
    return mx, mean


def dev(a, dtype: str = "f32"):
    """numpy float array whose values are exactly representable in `dtype` -> CUDA tensor."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(TORCH_DT[dtype]).cuda()


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(F64)


def bits(t):
    """Raw storage bits of a CUDA tensor, for bit-exact comparisons."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy()
    return t.cpu().numpy()


class DeviceWorkload:
    """A workload's inputs on the GPU, produced by the shared generator (same values the
    oracle regenerates on the host)."""

    def __init__(self, w: mi.Workload):
        self.w = w
        dt = TORCH_DT[w.dtype]
        self.x = torch.empty((w.T, w.d), dtype=dt, device="cuda")
        mi.randn_torch(w.seed, mi.X, 0, w.T, w.d, w.sigma_x, w.dtype, "cuda", out=self.x)
        self.w_router = torch.empty((w.E, w.d), dtype=dt, device="cuda")
        mi.randn_torch(w.seed, mi.W_ROUTER, 0, w.E, w.d, w.sigma_w, w.dtype, "cuda", out=self.w_router)
        b = mi.expert_bias(w)
        self.bias = None if b is None else torch.from_numpy(b).cuda()
        n = w.E + (1 if w.shared_f else 0)
        self.w_gu = torch.empty((n, 2 * w.f, w.d), dtype=dt, device="cuda")
        self.w_down = torch.empty((n, w.d, w.f), dtype=dt, device="cuda")
        mi.fill_weights_torch(w, self.w_gu, self.w_down, "cuda")
        torch.cuda.synchronize()

    def free(self):
        for a in ("x", "w_router", "bias", "w_gu", "w_down"):
            setattr(self, a, None)
        torch.cuda.empty_cache()
