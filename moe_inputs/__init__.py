"""Seeded synthetic inputs for the dropless MoE layer.

This module is shared by the tests, the benchmark and the oracle's checks, and it holds
none of the layer's arithmetic: no routing, no permutation, no GEMM, no rounding rule of
the method. It only turns (seed, tensor id, slab id, element index) into a value, through
an integer hash and a lookup into a table of normal quantiles, and it describes the
workloads (layer shapes, routing score, expert-bias recipe).

Why a hash and a table instead of a library RNG: the same element must come out
bit-identical on the host (numpy, for the oracle, which may need only a few rows of one
expert's weights) and on the device (torch, for the GPU path, which needs all 22.5 GB of
DeepSeek-V3-shaped expert weights in well under a second). The hash uses only xor, shifts
and products of 32-bit values by constants below 2**31, so every intermediate fits in a
signed 64-bit integer and numpy and torch compute the same bits. The top 16 bits of the
hash index a 65,536-entry table of N(0, 1) quantiles (midpoint rule), scaled by sigma and
rounded once to the storage dtype. The result is a normal distribution truncated at about
4.3 sigma and quantised to 65,536 levels before the storage rounding, which bf16 cannot
resolve anyway.
"""
from __future__ import annotations

import dataclasses
import functools
import math
from typing import Optional

import numpy as np

MASK32 = 0xFFFFFFFF
_M1 = 0x7FEB352D
_M2 = 0x2C1B3C6D
_M3 = 0x297A2D39

# tensor ids of the key derivation
X, W_ROUTER, W_GATE, W_UP, W_DOWN, SHARED, D_OUT = 0, 1, 3, 4, 5, 6, 7
D_TOPK_W = 8   # the gradient reaching the routing weights, for the router backward alone


def _mix(x):
    """32-bit avalanche mix on non-negative int64 values (numpy, torch or Python int)."""
    x = x ^ (x >> 16)
    x = (x * _M1) & MASK32
    x = x ^ (x >> 15)
    x = (x * _M2) & MASK32
    x = x ^ (x >> 16)
    x = (x * _M3) & MASK32
    x = x ^ (x >> 15)
    return x


def slab_key(seed: int, tensor: int, slab: int = 0) -> tuple[int, int]:
    """Two 32-bit keys for one slab (one expert's matrix, or a whole activation)."""
    a = _mix((seed * 0x9E3779B1 + 0x632BE5AB) & MASK32)
    a = _mix(a ^ ((tensor * 0x2545F491) & MASK32))
    a = _mix(a ^ ((slab * 0x68E31DA4 + 0x1B56C4E9) & MASK32))
    b = _mix(a ^ 0x5BD1E995)
    return a, b


def _hash_top16(counter, key: tuple[int, int]):
    h = _mix((counter + key[0]) & MASK32)
    h = _mix(h ^ key[1])
    return h >> 16


@functools.lru_cache(maxsize=None)
def _quantiles() -> np.ndarray:
    from scipy.special import ndtri
    p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return ndtri(p)


@functools.lru_cache(maxsize=None)
def normal_table(sigma: float, dtype: str) -> np.ndarray:
    """The 65,536 values one element can take, as float32 holding exactly the stored value.

    dtype "bf16": sigma * quantile rounded to float32, then to bfloat16 (nearest-even, via
    torch); dtype "f32": rounded to float32 only.
    """
    import torch
    v = torch.from_numpy(_quantiles() * sigma).to(torch.float32)
    if dtype == "bf16":
        v = v.to(torch.bfloat16).to(torch.float32)
    elif dtype != "f32":
        raise ValueError(dtype)
    return v.numpy().copy()


def randn_np(seed: int, tensor: int, slab: int, rows, cols: int, sigma: float, dtype: str,
             col_index=None) -> np.ndarray:
    """Rows `rows` (an int count, or an index array) of a [*, cols] slab, as float32; with
    `col_index`, only those columns."""
    if isinstance(rows, (int, np.integer)):
        rows = np.arange(int(rows), dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    assert rows.size == 0 or (int(rows.max()) + 1) * cols <= 2 ** 32
    cidx = np.arange(cols, dtype=np.int64) if col_index is None else np.asarray(col_index, dtype=np.int64)
    counter = rows[:, None] * cols + cidx[None, :]
    idx = _hash_top16(counter, slab_key(seed, tensor, slab))
    return normal_table(sigma, dtype)[idx]


def randn_torch(seed: int, tensor: int, slab: int, rows: int, cols: int, sigma: float, dtype: str,
                device, out=None):
    """The same values as `randn_np(..., rows, ...)`, produced by torch on `device`.

    Writes into `out` (a [rows, cols] tensor view) when given; generation is chunked so the
    int64 temporaries stay small.
    """
    import torch
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    assert rows * cols <= 2 ** 32
    table = torch.from_numpy(normal_table(sigma, dtype)).to(device=device, dtype=tdt)
    if out is None:
        out = torch.empty((rows, cols), dtype=tdt, device=device)
    flat = out.view(-1)
    key = slab_key(seed, tensor, slab)
    n = rows * cols
    step = 1 << 25
    for s in range(0, n, step):
        e = min(n, s + step)
        c = torch.arange(s, e, dtype=torch.int64, device=device)
        flat[s:e] = table[_hash_top16(c, key)]
    return out


def randint_np(seed: int, tensor: int, slab: int, rows, cols: int, lo: int, hi: int, scale_log2: int) -> np.ndarray:
    """Integers uniform in [lo, hi] times 2**scale_log2 (float32), from the same hash as
    `randn_np`; `randint_torch` gives the same values on the device."""
    if isinstance(rows, (int, np.integer)):
        rows = np.arange(int(rows), dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    counter = rows[:, None] * cols + np.arange(cols, dtype=np.int64)[None, :]
    h = _hash_top16(counter, slab_key(seed, tensor, slab))
    return ((h % (hi - lo + 1) + lo).astype(np.float64) * math.ldexp(1.0, scale_log2)).astype(np.float32)


def randint_torch(seed: int, tensor: int, slab: int, rows: int, cols: int, lo: int, hi: int, scale_log2: int,
                  dtype: str, device, out=None):
    import torch
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    if out is None:
        out = torch.empty((rows, cols), dtype=tdt, device=device)
    flat = out.view(-1)
    key = slab_key(seed, tensor, slab)
    n = rows * cols
    step = 1 << 25
    for s in range(0, n, step):
        e = min(n, s + step)
        c = torch.arange(s, e, dtype=torch.int64, device=device)
        v = (_hash_top16(c, key) % (hi - lo + 1) + lo).to(torch.float32) * math.ldexp(1.0, scale_log2)
        flat[s:e] = v.to(tdt)
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """One MoE layer shape and its synthetic-input recipe."""
    name: str
    T: int                      # tokens
    d: int                      # hidden size
    f: int                      # expert FFN width
    E: int                      # routed experts
    k: int                      # experts per token
    dtype: str                  # "f32" or "bf16" storage of activations and weights
    score: str                  # "softmax" or "sigmoid"
    bias: Optional[tuple]       # None | ("linear", beta) | ("zipf", s, lam)
    shared_f: int = 0           # FFN width of the always-on shared expert (0 = none)
    seed: int = 0
    sigma_x: float = 1.0
    sigma_w: float = 0.02
    mxfp8: bool = False
    backward: bool = False
    mxfp4: bool = False


WORKLOADS = {
    # the five layer shapes the method is exercised on
    "tiny": Workload("tiny", 64, 128, 256, 8, 2, "f32", "softmax", None, 0, seed=0),
    "mixtral": Workload("mixtral", 4096, 4096, 14336, 8, 2, "bf16", "softmax", ("linear", 1.0), 0, seed=1),
    "qwen3": Workload("qwen3", 8192, 4096, 1536, 128, 8, "bf16", "softmax", ("zipf", 1.0, 1.6), 0, seed=2),
    "dsv3": Workload("dsv3", 8192, 7168, 2048, 256, 8, "bf16", "sigmoid", ("zipf", 1.2, 1.0), 2048, seed=3),
    "dsv3_mxfp8": Workload("dsv3_mxfp8", 8192, 7168, 2048, 256, 8, "bf16", "sigmoid", ("zipf", 1.2, 1.0), 2048,
                           seed=3, mxfp8=True, backward=True),
    # one GPU's share of the DeepSeek-V3 layer under 8-way expert parallelism: 32 local experts
    # receiving 65,536 rows (about 2,048 each, the compute-bound regime), plus the GPU's own
    # shared expert over its 8,192 tokens; the dispatch that would deliver those rows from the
    # other GPUs is replaced by routing 8,192 local tokens 8 ways over the 32 experts
    # the DeepSeek-V3 layer forward with MXFP4 expert GEMMs (d and f multiples of 256)
    "dsv3_mxfp4": Workload("dsv3_mxfp4", 8192, 7168, 2048, 256, 8, "bf16", "sigmoid", ("zipf", 1.2, 1.0), 2048,
                           seed=3, mxfp4=True),
    "dsv3_ep8": Workload("dsv3_ep8", 8192, 7168, 2048, 32, 8, "bf16", "sigmoid", None, 2048, seed=4),
    # reduced shapes the oracle finishes in seconds: several tiles, ragged tails, empty and
    # one-row groups, one hot group
    "small_softmax": Workload("small_softmax", 1000, 256, 384, 16, 4, "bf16", "softmax", ("zipf", 1.0, 1.0), 0, seed=11),
    "small_sigmoid": Workload("small_sigmoid", 777, 320, 192, 24, 6, "bf16", "sigmoid", ("zipf", 1.2, 0.7), 192, seed=12),
    # the MXFP8 training step at a reduced shape (d, f multiples of 128 as its GEMMs need)
    "small_mxfp8": Workload("small_mxfp8", 600, 384, 256, 12, 3, "bf16", "sigmoid", ("zipf", 1.2, 0.7), 256,
                            seed=13, mxfp8=True, backward=True),
    # the MXFP8 step with contraction lengths of 1024 or more in every forward and data-gradient
    # GEMM, still small enough for the oracle to finish in seconds
    "mid_mxfp8": Workload("mid_mxfp8", 1024, 1024, 1024, 8, 2, "bf16", "sigmoid", ("zipf", 1.2, 0.7), 1024,
                          seed=21, mxfp8=True, backward=True),
    # the MXFP4 forward at a reduced shape
    "small_mxfp4": Workload("small_mxfp4", 600, 512, 256, 12, 3, "bf16", "sigmoid", ("zipf", 1.2, 0.7), 256,
                            seed=14, mxfp4=True),
}


def expert_bias(w: Workload) -> Optional[np.ndarray]:
    """Per-expert logit bias [E] float32 for the workload's skew recipe (None: no bias).

    linear: beta * (e / (E - 1) - 1/2), a mild monotone skew.
    zipf:   -lam * s * ln(rank(e)), rank(e) in 1..E a seeded permutation of the experts, so
            exp(bias) follows a Zipf(s) law over expert rank; lam scales its strength.
    dead:   -30 on a seeded set of n experts, 0 elsewhere: those experts are never selected
            while at least k others remain (forced empty groups).
    """
    if w.bias is None:
        return None
    kind = w.bias[0]
    e = np.arange(w.E, dtype=np.float64)
    if kind == "linear":
        b = w.bias[1] * (e / max(w.E - 1, 1) - 0.5)
    elif kind == "zipf":
        s, lam = w.bias[1], w.bias[2]
        rank = np.random.Generator(np.random.PCG64(w.seed + 1000)).permutation(w.E) + 1
        b = -lam * s * np.log(rank.astype(np.float64))
    elif kind == "dead":
        dead = np.random.Generator(np.random.PCG64(w.seed + 1000)).permutation(w.E)[:w.bias[1]]
        b = np.zeros(w.E)
        b[dead] = -30.0
    else:
        raise ValueError(kind)
    return b.astype(np.float32)


def fuzz_workloads(n: int = 14, seed: int = 4242) -> list:
    """A seeded sweep of layer shapes over the edges the method has: E in 1..256, k in
    1..min(8, E), T in 1..9000 (log-uniform), softmax or sigmoid, with or without a shared
    expert, skew-free, Zipf-skewed or with a forced set of experts that receive nothing (empty
    groups); d and f multiples of 64; group sizes fall anywhere, mostly not multiples of 32.
    One in seven shapes is fp32. Sizes stay small enough for the oracle to finish in seconds."""
    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    for i in range(n):
        E = int(g.choice([1, 2, 3, 5, 8, 13, 32, 64, 100, 128, 200, 256]))
        k = int(g.integers(1, min(8, E) + 1))
        T = int(round(math.exp(g.uniform(0.0, math.log(9000.0)))))
        d = int(g.choice([64, 128, 192, 320, 512]))
        f = int(g.choice([64, 128, 192, 256, 384]))
        if T * k * d * f > 2e9:                       # keep the oracle's work to a few seconds
            f = 64
        score = "softmax" if g.integers(0, 2) == 0 else "sigmoid"
        kind = int(g.integers(0, 3))
        if kind == 1:
            bias = ("zipf", float(g.uniform(0.8, 1.4)), float(g.uniform(0.5, 2.0)))
        elif kind == 2 and E - k >= 1:
            bias = ("dead", int(g.integers(1, E - k + 1)))
        else:
            bias = None
        shared = f if g.integers(0, 2) == 0 else 0
        dtype = "f32" if i % 7 == 6 else "bf16"
        out.append(Workload(f"fuzz{i}", T, d, f, E, k, dtype, score, bias, shared, seed=100 + i))
    # the ends of the ranges: one expert taking all 9000 tokens; one token; 256 experts with
    # most of them dead, on the router's split-K path (T >= 256, E % 8 == 0, d % 256 == 0)
    out.append(Workload("fuzz_e1", 9000, 128, 128, 1, 1, "bf16", "softmax", None, 0, seed=201))
    out.append(Workload("fuzz_t1", 1, 64, 64, 64, 8, "bf16", "sigmoid", None, 64, seed=202))
    out.append(Workload("fuzz_wide", 3000, 512, 128, 256, 8, "bf16", "sigmoid", ("dead", 200), 128, seed=203))
    return out


def x_np(w: Workload, rows=None) -> np.ndarray:
    return randn_np(w.seed, X, 0, w.T if rows is None else rows, w.d, w.sigma_x, w.dtype)


def w_router_np(w: Workload) -> np.ndarray:
    """Router weight [E, d]: row e is expert e's router vector."""
    return randn_np(w.seed, W_ROUTER, 0, w.E, w.d, w.sigma_w, w.dtype)


def w_gate_up_np(w: Workload, e: int) -> np.ndarray:
    """Expert e's [2f, d] gate/up weight: rows 0..f-1 gate, rows f..2f-1 up (shared: e = E)."""
    if e == w.E:
        g = randn_np(w.seed, SHARED, 0, w.shared_f, w.d, w.sigma_w, w.dtype)
        u = randn_np(w.seed, SHARED, 1, w.shared_f, w.d, w.sigma_w, w.dtype)
    else:
        g = randn_np(w.seed, W_GATE, e, w.f, w.d, w.sigma_w, w.dtype)
        u = randn_np(w.seed, W_UP, e, w.f, w.d, w.sigma_w, w.dtype)
    return np.concatenate([g, u], axis=0)


def w_down_np(w: Workload, e: int) -> np.ndarray:
    """Expert e's [d, f] down weight (shared: e = E)."""
    if e == w.E:
        return randn_np(w.seed, SHARED, 2, w.d, w.shared_f, w.sigma_w, w.dtype)
    return randn_np(w.seed, W_DOWN, e, w.d, w.f, w.sigma_w, w.dtype)


def d_out_np(w: Workload) -> np.ndarray:
    return randn_np(w.seed, D_OUT, 0, w.T, w.d, 1.0, w.dtype)


def fill_weights_torch(w: Workload, w_gu, w_down, device):
    """Fill stacked device weights: w_gu [E(+1), 2f, d], w_down [E(+1), d, f]; slot E is the
    shared expert when the workload has one (it needs shared_f == f)."""
    n = w.E + (1 if w.shared_f else 0)
    if w.shared_f:
        assert w.shared_f == w.f
    for e in range(n):
        if e == w.E:
            randn_torch(w.seed, SHARED, 0, w.f, w.d, w.sigma_w, w.dtype, device, out=w_gu[e, :w.f])
            randn_torch(w.seed, SHARED, 1, w.f, w.d, w.sigma_w, w.dtype, device, out=w_gu[e, w.f:])
            randn_torch(w.seed, SHARED, 2, w.d, w.f, w.sigma_w, w.dtype, device, out=w_down[e])
        else:
            randn_torch(w.seed, W_GATE, e, w.f, w.d, w.sigma_w, w.dtype, device, out=w_gu[e, :w.f])
            randn_torch(w.seed, W_UP, e, w.f, w.d, w.sigma_w, w.dtype, device, out=w_gu[e, w.f:])
            randn_torch(w.seed, W_DOWN, e, w.d, w.f, w.sigma_w, w.dtype, device, out=w_down[e])


def integer_valued(shape, lo: int, hi: int, scale_log2: int, seed: int) -> np.ndarray:
    """Small integers in [lo, hi] times 2**scale_log2, as float32: products and partial sums
    of such values are exact in fp32 as long as they stay below 2**24 in units of the scale."""
    g = np.random.Generator(np.random.PCG64(seed))
    v = g.integers(lo, hi + 1, size=shape).astype(np.float64) * math.ldexp(1.0, scale_log2)
    return v.astype(np.float32)
