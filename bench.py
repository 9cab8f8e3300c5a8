"""Benchmark: one dropless MoE layer forward (route -> permute -> grouped SwiGLU MLP ->
combine) on one MI355X, DeepSeek-V3-shaped bf16 by default.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3] [--no-cpu-baseline]

Prints ONE JSON line. `value` is useful GEMM FLOPs (6*T*k*d*f + 6*T*d*f_shared, padding never
counted, router projection excluded) divided by the whole step time, i.e. layer TFLOPS;
`gemm_tflops` uses the two grouped-GEMM launches' own event time instead, `tokens_per_s` is
T / step time. Inputs and weights are resident in HBM before timing starts.

--workload dsv3_mxfp8 times the MXFP8 training step instead: the per-step quantisation of
the weights (both axis copies), the forward and the backward of the experts, permutation and
combine (18*(T*k + T)*d*f useful FLOPs); `value` covers the whole step, `ms_without_weight_quant`
and `value_without_weight_quant` leave the weight quantisation out.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
FP4_PEAK_TFLOPS = 10100.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--materialise-gather", action="store_true",
                    help="write x_perm in the permute and read it in GEMM 1 (default: gather fused into GEMM 1)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run a 1 GiB device copy (torch.neg into a second buffer) three "
                         "times, so a counter pass of this same command sees the HBM bytes of a copy of known size")
    return ap.parse_args()


COPY_CAL_BYTES = 1 << 30
GEMM_SOURCES = ("dropless_mixture_experts_device_amd/csrc/gemm.hip",
                "dropless_mixture_experts_device_amd/csrc/moe_internal.h")


def gemm_source_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def pmc_traffic(workload, kernel="gemm1_swiglu"):
    """HBM bytes per launch of one GEMM kernel (the bf16 gate/up GEMM, or an MXFP8 step's
    dominant GEMM) from the committed counter summary (FETCH_SIZE and WRITE_SIZE passes, each
    scaled by the same counter's reading for a copy of known size). None when no summary
    exists or the GEMM sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                key, val = line[2:].split(":", 1)
                fields[key.strip()] = val.strip().strip("`")
    if fields.get("source_sha256") != gemm_source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy(dev):
    """A plain 1 GiB copy (torch.neg into a second buffer), three times, so a counter pass of
    the same command sees the HBM bytes of a copy of known size."""
    import torch
    src = torch.zeros((COPY_CAL_BYTES // 2,), dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


FLUSH_BYTES = 1 << 30   # written between timed steps: twice the 256 MB MALL plus every XCD's L2


class CacheFlush:
    """A 1 GiB device buffer read once (a sum over it) before each timed step, outside the timing
    events, so no step starts with its inputs or weights left in L2 or the MALL by the step before
    it. A read rather than a write: the lines it leaves behind are clean, so no write-back of the
    flush itself spills into the timed step, and the previous step's dirty lines are written back
    during the flush."""

    def __init__(self, dev):
        import torch
        self.buf = torch.ones((FLUSH_BYTES // 4,), dtype=torch.int32, device=dev)
        self.sink = None

    def __call__(self):
        self.sink = self.buf.sum()


def spread(v):
    """Median, 10th and 90th percentile of per-step times (ms)."""
    a = np.asarray(v, np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def host_info():
    """CPU model (from /proc/cpuinfo) and the BLAS numpy is built against."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        cfg = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{cfg.get('name')} {cfg.get('version')}"
    except Exception:
        pass
    try:
        ncpu = len(os.sched_getaffinity(0))
    except Exception:
        ncpu = os.cpu_count()
    return {"cpu_model": model, "blas": blas, "cpus_available": ncpu}


def time_graph(step, steps, flush):
    """The step captured once in a HIP graph, then `steps` replays, each after a cache flush,
    timed with events around the replay on the launching stream. Returns per-replay ms."""
    import torch
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        flush()
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    out = [e0.elapsed_time(e1) for e0, e1 in ev]
    del g
    return out


def useful_flops(w, counts):
    routed = 6.0 * w.T * w.k * w.d * w.f
    shared = 6.0 * w.T * w.d * w.shared_f
    return routed + shared


def gemm1_bytes(w, counts, fused):
    """Algorithmic HBM bytes of grouped GEMM 1 (gate/up + SwiGLU): the gate/up weights of
    every non-empty routed group and of the shared expert once, the A rows once (x itself when the gather is fused, else
    x_perm), H written once, plus the index metadata."""
    nonempty = int(np.count_nonzero(counts))
    rows = w.T * w.k + (w.T if w.shared_f else 0)
    wbytes = nonempty * 2 * w.f * w.d * 2 + (2 * w.shared_f * w.d * 2 if w.shared_f else 0)
    abytes = (w.T * w.d * 2) if fused else rows * w.d * 2
    hbytes = rows * w.f * 2
    return wbytes + abytes + hbytes + rows * 4


CPU_BUDGET_S = 25.0


def cpu_baseline(w, w_gu_dev, w_down_dev, mx4=False):
    """The oracle's forward (fp64 numpy, as it stands) on the host cores: routing, the
    permutation and gather of all T tokens, then the SwiGLU experts one group at a time in a
    spread order (0, 16, 32, ..., then 8, 24, ...), the shared expert on all tokens, and the
    combine, until about CPU_BUDGET_S seconds of oracle time are spent. Each expert's weights
    are copied off the GPU (same generator, same values) outside the timed region. Reported
    in useful TFLOPS of the groups it finished. mx4: the oracle's MXFP4 forward (every GEMM
    operand through its row-wise MXFP4 quantiser, the weights' quantisation included)."""
    import moe_inputs as mi
    from oracle import moe_oracle as O
    try:
        import threadpoolctl
        cores = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        cores = os.cpu_count() or 1
    x = mi.x_np(w)
    wr = mi.w_router_np(w)
    bias = mi.expert_bias(w)
    spent = 0.0
    t0 = time.perf_counter()
    idx, wt, _ = O.route(x, wr, bias, w.k, w.score)
    off, row_of, src = O.permutation(idx, w.E, w.T if w.shared_f else 0)
    xp = O.gather_rows(x, src)
    spent += time.perf_counter() - t0
    Y = np.zeros((int(off[-1]), w.d))
    groups = ([w.E] if w.shared_f else []) + [e for r in range(16) for e in range(int(f"{r:04b}"[::-1], 2), w.E, 16)]
    flops, done = 0.0, 0
    for g in groups:
        if spent >= CPU_BUDGET_S:
            break
        lo, hi = int(off[g]), int(off[g + 1])
        done += 1
        if hi == lo:
            continue
        gu = w_gu_dev[g].float().cpu().numpy()
        dn = w_down_dev[g].float().cpu().numpy()
        t0 = time.perf_counter()
        _, Y[lo:hi] = O.expert_forward(xp[lo:hi], gu, dn, O.round_bf16, mx4=mx4)
        spent += time.perf_counter() - t0
        flops += 6.0 * (hi - lo) * w.d * (gu.shape[0] // 2)
    whole = done == len(groups)
    if whole:
        t0 = time.perf_counter()
        O.combine(Y[:w.T * w.k], wt, row_of, Y[w.T * w.k:] if w.shared_f else None, O.round_bf16)
        spent += time.perf_counter() - t0
    what = ("the whole layer forward" if whole else
            f"routing, permutation and gather of all {w.T} tokens, then {done} of {len(groups)} expert groups "
            f"(shared first, then ids in the order 0,16,32,...,8,24,...) on their real rows, stopped at "
            f"{CPU_BUDGET_S:.0f} s; no combine")
    return {"value": flops / spent / 1e12, "unit": "TFLOPS", "cores": int(cores), "kind": "oracle",
            "seconds": round(spent, 2), "host": host_info(),
            "sample": f"fp64 numpy {'MXFP4 ' if mx4 else ''}oracle on {what}; value = useful FLOPs of the "
                      f"finished groups / oracle time"}


def mx_gemm_work(w, rows, nonempty):
    """Algorithmic HBM bytes and FLOPs of each MXFP8 GEMM of the step: E4M3 operands with one
    scale byte per 32 elements read once (weights of non-empty groups only), bf16 outputs
    written once; GEMM 1 writes the saved gate/up pre-activations and H's two MXFP8 copies
    (row-wise and column-wise, quantised in its epilogue) instead of a bf16 H; dgrad 2 reads
    the saved pre-activations and writes dGU's two MXFP8 copies (the SwiGLU backward in its
    epilogue) instead of a bf16 dH."""
    d, f, G = w.d, w.f, w.E + (1 if w.shared_f else 0)
    q = 33.0 / 32.0
    return {
        "gemm1_swiglu": (nonempty * 2 * f * d * q + w.T * d * q + 2 * rows * f * q + rows * 2 * f * 2 + rows * 4,
                         2.0 * rows * d * 2 * f),
        "gemm2": (nonempty * d * f * q + rows * f * q + rows * d * 2, 2.0 * rows * f * d),
        "dgrad2": (nonempty * f * d * q + rows * d * q + rows * 2 * f * 2 + 2 * rows * 2 * f * q, 2.0 * rows * d * f),
        "wgrad2": ((d + f) * rows * q + G * d * f * 2, 2.0 * rows * d * f),
        "dgrad1": (nonempty * d * 2 * f * q + rows * 2 * f * q + rows * d * 2, 2.0 * rows * 2 * f * d),
        "wgrad1": ((2 * f + d) * rows * q + G * 2 * f * d * 2, 2.0 * rows * 2 * f * d),
    }


def cpu_baseline_mx(w, w_gu_dev, w_down_dev):
    """The oracle's MXFP8 step (fp64 numpy on dequantised MX operands, as it stands): routing
    and the permutation of all tokens, then each group's MX forward and backward in the same
    spread order as the bf16 baseline until about CPU_BUDGET_S seconds of oracle time."""
    import moe_inputs as mi
    from oracle import moe_oracle as O
    try:
        import threadpoolctl
        cores = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        cores = os.cpu_count() or 1
    x = mi.x_np(w)
    spent = 0.0
    t0 = time.perf_counter()
    wr = mi.w_router_np(w)
    idx, wt, keys = O.route(x, wr, mi.expert_bias(w), w.k, w.score)
    off, row_of, src = O.permutation(idx, w.E, w.T if w.shared_f else 0)
    # the router's backward for every token (the step runs it; its FLOPs are not counted)
    g_w = mi.randn_np(w.seed, mi.D_TOPK_W, 0, w.T, w.k, 1.0, "f32")
    O.router_backward(x, wr, O.topk_weights_backward(keys, idx, g_w, w.score))
    spent += time.perf_counter() - t0
    groups = ([w.E] if w.shared_f else []) + [e for r in range(16) for e in range(int(f"{r:04b}"[::-1], 2), w.E, 16)]
    flops, done = 0.0, 0
    for g in groups:
        if spent >= CPU_BUDGET_S:
            break
        lo, hi = int(off[g]), int(off[g + 1])
        done += 1
        if hi == lo:
            continue
        gu = w_gu_dev[g].float().cpu().numpy()
        dn = w_down_dev[g].float().cpu().numpy()
        dY = mi.randn_np(w.seed, mi.D_OUT, 0, src[lo:hi], w.d, 1.0, "bf16")
        t0 = time.perf_counter()
        O.expert_backward(x[src[lo:hi]], gu, dn, dY, O.round_bf16, mx=True)   # recomputes the forward
        spent += time.perf_counter() - t0
        flops += 18.0 * (hi - lo) * w.d * (gu.shape[0] // 2)
    return {"value": flops / spent / 1e12, "unit": "TFLOPS", "cores": int(cores), "kind": "oracle",
            "seconds": round(spent, 2), "host": host_info(),
            "sample": f"fp64 numpy MX oracle: routing, permutation and the router's backward of all {w.T} tokens, "
                      f"then the MXFP8 forward "
                      f"and backward of {done} of {len(groups)} expert groups (shared first, then ids "
                      f"0,16,32,...,8,24,...) on their real rows, stopped at {CPU_BUDGET_S:.0f} s; value = useful "
                      f"FLOPs (18 m d f per group) of the finished groups / oracle time"}


def main_mx(args, w):
    import torch
    import moe_inputs as mi
    from dropless_mixture_experts_device_amd import _lib as L
    from dropless_mixture_experts_device_amd import layer

    torch.cuda.init()
    dev = "cuda"
    x = torch.empty((w.T, w.d), dtype=torch.bfloat16, device=dev)
    mi.randn_torch(w.seed, mi.X, 0, w.T, w.d, w.sigma_x, w.dtype, dev, out=x)
    wr = torch.empty((w.E, w.d), dtype=torch.bfloat16, device=dev)
    mi.randn_torch(w.seed, mi.W_ROUTER, 0, w.E, w.d, w.sigma_w, w.dtype, dev, out=wr)
    b0 = mi.expert_bias(w)
    bias = None if b0 is None else torch.from_numpy(b0).to(dev)
    n = w.E + (1 if w.shared_f else 0)
    w_gu = torch.empty((n, 2 * w.f, w.d), dtype=torch.bfloat16, device=dev)
    w_down = torch.empty((n, w.d, w.f), dtype=torch.bfloat16, device=dev)
    mi.fill_weights_torch(w, w_gu, w_down, dev)
    d_out = mi.randn_torch(w.seed, mi.D_OUT, 0, w.T, w.d, 1.0, "bf16", dev)
    s = layer.LayerShape(T=w.T, d=w.d, f=w.f, E=w.E, k=w.k, shared=bool(w.shared_f),
                         score=L.MOE_SOFTMAX if w.score == "softmax" else L.MOE_SIGMOID)
    mw = layer.MxWeights(s, dev)
    b = layer.MxBuffers(s, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step(rec=None):
        mark = None
        if rec is not None:
            def mark(name):
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                rec.append((name, e))
            mark("start")
        mw.quantise(w_gu, w_down)
        if mark:
            mark("weight_quant")
        layer.forward_mx(x, wr, bias, mw, s, b, mark=mark, write_h=False)
        layer.backward_mx(x, d_out, mw, s, b, mark=mark, w_router=wr)

    flush = CacheFlush(dev)
    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    recs = [[] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        step(recs[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    names = [n for n, _ in recs[0][1:]]
    per = np.array([[r[j][1].elapsed_time(r[j + 1][1]) for j in range(len(r) - 1)] for r in recs])
    pm = dict(zip(names, np.median(per, axis=0)))
    step_all = np.array([r[0][1].elapsed_time(r[-1][1]) for r in recs])
    ms = float(np.median(step_all))
    graph_ms = time_graph(step, args.steps, flush)
    counts = np.diff(b.offsets.cpu().numpy())[:w.E]
    rows = s.rows
    flops = 18.0 * rows * w.d * w.f
    nonempty = int(np.count_nonzero(counts)) + (1 if w.shared_f else 0)
    work = mx_gemm_work(w, rows, nonempty)
    dom = max(work, key=lambda k: pm[k])
    by, fl = work[dom]
    t = pm[dom] * 1e-3
    t_hbm, t_mfma = by / (HBM_PEAK_GBS * 1e9), fl / (FP8_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(by / t / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(fl / t / 1e12, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(fl / t / 1e12 / FP8_PEAK_TFLOPS, 4)}
    roof.update({"traffic": pmc_traffic(w.name, dom), "kernel": f"moe_grouped_gemm MXFP8 {dom}", "algorithmic_bytes": int(by),
                 "algorithmic_flops": fl, "ms": round(pm[dom], 4)})
    no_wq = ms - pm["weight_quant"]
    gemm_ms = sum(pm[k] for k in work)
    res = {
        "metric": "MoE layer fwd+bwd TFLOPS (useful FLOPs) + tokens/s, DSv3-shaped MXFP8 training step",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3 (MXFP8, E8M0/32)",
        "data": "synthetic (seeded hash-table normal inputs and output gradient, Zipf expert-bias skew; "
                "random-init weights)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "f": w.f, "E": w.E, "k": w.k, "score": w.score,
                   "shared_f": w.shared_f, "groups_nonempty": int(np.count_nonzero(counts)),
                   "group_max": int(counts.max()), "group_min": int(counts.min()),
                   "groups_empty": int((counts == 0).sum())},
        "timing": ("median over the timed steps of HIP events on the launching stream; every timed step "
                   f"starts after a {FLUSH_BYTES >> 20} MiB read of a scratch buffer outside the events"),
        "step_ms": spread(step_all),
        "wall_ms_per_step_incl_flush": round(wall_ms, 4),
        "graph_ms_per_step": spread(graph_ms),
        "tokens_per_s": round(w.T / (ms * 1e-3), 1),
        "ms_without_weight_quant": round(no_wq, 4),
        "value_without_weight_quant": round(flops / (no_wq * 1e-3) / 1e12, 2),
        "gemm_tflops": round(flops / (gemm_ms * 1e-3) / 1e12, 2),
        "stage_ms": {k: spread(per[:, j]) for j, k in enumerate(names)},
        "gemm_tflops_by_stage": {k: round(work[k][1] / (pm[k] * 1e-3) / 1e12, 1) for k in work},
        "gemm_gbs_by_stage": {k: round(work[k][0] / (pm[k] * 1e-3) / 1e9, 1) for k in work},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if args.calibrate_copy:
        calibrate_copy(dev)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_mx(w, w_gu, w_down)
    print(json.dumps(res), flush=True)


def mx4_gemm_work(w, rows, nonempty):
    """Algorithmic HBM bytes and FLOPs of the two MXFP4 GEMMs of the forward: E2M1 operands at
    half a byte per element plus one scale byte per 32 (weights of non-empty groups and the
    shared expert once, x once through the fused gather), GEMM 1's output as the MXFP4 codes
    its epilogue writes, GEMM 2's bf16 output once, the gather index read once."""
    d, f = w.d, w.f
    q = 0.5 + 1.0 / 32.0
    return {
        "gemm1_swiglu": (nonempty * 2 * f * d * q + w.T * d * q + rows * f * q + rows * 4, 2.0 * rows * d * 2 * f),
        "gemm2": (nonempty * d * f * q + rows * f * q + rows * d * 2, 2.0 * rows * f * d),
    }


def main_mx4(args, w):
    """The MXFP4 layer forward. The expert weights are quantised once before the timed steps
    (a forward-only layer's weights do not change between calls); x and H are quantised
    inside every step."""
    import torch
    import moe_inputs as mi
    from dropless_mixture_experts_device_amd import _lib as L
    from dropless_mixture_experts_device_amd import layer

    torch.cuda.init()
    dev = "cuda"
    x = torch.empty((w.T, w.d), dtype=torch.bfloat16, device=dev)
    mi.randn_torch(w.seed, mi.X, 0, w.T, w.d, w.sigma_x, w.dtype, dev, out=x)
    wr = torch.empty((w.E, w.d), dtype=torch.bfloat16, device=dev)
    mi.randn_torch(w.seed, mi.W_ROUTER, 0, w.E, w.d, w.sigma_w, w.dtype, dev, out=wr)
    b0 = mi.expert_bias(w)
    bias = None if b0 is None else torch.from_numpy(b0).to(dev)
    n = w.E + (1 if w.shared_f else 0)
    w_gu = torch.empty((n, 2 * w.f, w.d), dtype=torch.bfloat16, device=dev)
    w_down = torch.empty((n, w.d, w.f), dtype=torch.bfloat16, device=dev)
    mi.fill_weights_torch(w, w_gu, w_down, dev)
    s = layer.LayerShape(T=w.T, d=w.d, f=w.f, E=w.E, k=w.k, shared=bool(w.shared_f),
                         score=L.MOE_SOFTMAX if w.score == "softmax" else L.MOE_SIGMOID)
    mw = layer.Mx4Weights(s, dev)
    b = layer.Mx4Buffers(s, dev)
    stream = torch.cuda.current_stream()
    # the weights' quantisation, timed on its own (not part of a step)
    mw.quantise(w_gu, w_down)
    q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    q0.record(stream)
    mw.quantise(w_gu, w_down)
    q1.record(stream)
    torch.cuda.synchronize()
    wq_ms = q0.elapsed_time(q1)

    def step(rec=None):
        mark = None
        if rec is not None:
            def mark(name):
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                rec.append((name, e))
            mark("start")
        layer.forward_mx4(x, wr, bias, mw, s, b, mark=mark, write_h=False)

    flush = CacheFlush(dev)
    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    recs = [[] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        step(recs[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    names = [nm for nm, _ in recs[0][1:]]
    per = np.array([[r[j][1].elapsed_time(r[j + 1][1]) for j in range(len(r) - 1)] for r in recs])
    pm = dict(zip(names, np.median(per, axis=0)))
    step_all = np.array([r[0][1].elapsed_time(r[-1][1]) for r in recs])
    ms = float(np.median(step_all))
    graph_ms = time_graph(step, args.steps, flush)
    counts = np.diff(b.offsets.cpu().numpy())[:w.E]
    flops = useful_flops(w, counts)
    nonempty = int(np.count_nonzero(counts)) + (1 if w.shared_f else 0)
    work = mx4_gemm_work(w, s.rows, nonempty)
    dom = max(work, key=lambda k: pm[k])
    by, fl = work[dom]
    t = pm[dom] * 1e-3
    t_hbm, t_mfma = by / (HBM_PEAK_GBS * 1e9), fl / (FP4_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(by / t / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(fl / t / 1e12, 1), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(fl / t / 1e12 / FP4_PEAK_TFLOPS, 4)}
    roof.update({"traffic": pmc_traffic(w.name, dom), "kernel": f"moe_grouped_gemm MXFP4 {dom}",
                 "algorithmic_bytes": int(by), "algorithmic_flops": fl, "ms": round(pm[dom], 4),
                 "mfma_frac": round(fl / t / 1e12 / FP4_PEAK_TFLOPS, 4),
                 "hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4)})
    gemm_ms = sum(pm[k] for k in work)
    res = {
        "metric": "MoE layer forward TFLOPS (useful FLOPs) + tokens/s, DSv3-shaped MXFP4 forward",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e2m1 (MXFP4, E8M0/32)",
        "data": "synthetic (seeded hash-table normal inputs, Zipf expert-bias skew; random-init weights)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "f": w.f, "E": w.E, "k": w.k, "score": w.score,
                   "shared_f": w.shared_f, "weights": "quantised to MXFP4 once, before the timed steps",
                   "groups_nonempty": int(np.count_nonzero(counts)), "group_max": int(counts.max()),
                   "group_min": int(counts.min()), "groups_empty": int((counts == 0).sum())},
        "timing": ("median over the timed steps of HIP events on the launching stream; every timed step "
                   f"starts after a {FLUSH_BYTES >> 20} MiB read of a scratch buffer outside the events"),
        "step_ms": spread(step_all),
        "wall_ms_per_step_incl_flush": round(wall_ms, 4),
        "graph_ms_per_step": spread(graph_ms),
        "tokens_per_s": round(w.T / (ms * 1e-3), 1),
        "weight_quant_ms": round(wq_ms, 4),
        "gemm_tflops": round(flops / (gemm_ms * 1e-3) / 1e12, 2),
        "stage_ms": {k: spread(per[:, j]) for j, k in enumerate(names)},
        "gemm_tflops_by_stage": {k: round(work[k][1] / (pm[k] * 1e-3) / 1e12, 1) for k in work},
        "gemm_gbs_by_stage": {k: round(work[k][0] / (pm[k] * 1e-3) / 1e9, 1) for k in work},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if args.calibrate_copy:
        calibrate_copy(dev)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, w_gu, w_down, mx4=True)
    print(json.dumps(res), flush=True)


# Workloads that were benchmarked together in one GPU run that ended in a GPU memory fault;
# which of them faulted, and why, is not known, so none of them is run until the cause is.
HELD_WORKLOADS = ("dsv3_ep8", "mixtral", "qwen3")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs on one GPU only (no collectives); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.workload in HELD_WORKLOADS:
        print(json.dumps({"error": f"workload {args.workload} is held: the first GPU run that included it "
                                   "ended in a GPU memory fault whose cause is not yet found",
                          "workload": args.workload}))
        sys.exit(3)
    import torch
    import moe_inputs as mi
    from dropless_mixture_experts_device_amd import _lib as L
    from dropless_mixture_experts_device_amd import layer

    w = mi.WORKLOADS[args.workload]
    if w.mxfp8:
        return main_mx(args, w)
    if w.mxfp4:
        return main_mx4(args, w)
    assert w.dtype == "bf16", "bench times the bf16 layer workloads"
    torch.cuda.init()
    dev = "cuda"
    x = torch.empty((w.T, w.d), dtype=torch.bfloat16, device=dev)
    mi.randn_torch(w.seed, mi.X, 0, w.T, w.d, w.sigma_x, w.dtype, dev, out=x)
    wr = torch.empty((w.E, w.d), dtype=torch.bfloat16, device=dev)
    mi.randn_torch(w.seed, mi.W_ROUTER, 0, w.E, w.d, w.sigma_w, w.dtype, dev, out=wr)
    b = mi.expert_bias(w)
    bias = None if b is None else torch.from_numpy(b).to(dev)
    n = w.E + (1 if w.shared_f else 0)
    w_gu = torch.empty((n, 2 * w.f, w.d), dtype=torch.bfloat16, device=dev)
    w_down = torch.empty((n, w.d, w.f), dtype=torch.bfloat16, device=dev)
    mi.fill_weights_torch(w, w_gu, w_down, dev)
    s = layer.LayerShape(T=w.T, d=w.d, f=w.f, E=w.E, k=w.k, shared=bool(w.shared_f),
                         score=L.MOE_SOFTMAX if w.score == "softmax" else L.MOE_SIGMOID)
    fused = not args.materialise_gather
    buf = layer.LayerBuffers(s, dev, fused_gather=fused)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    flush = CacheFlush(dev)
    STAGES = ("route", "permute", "gemm1_swiglu", "gemm2", "combine")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(args.steps)]

    def step(evs=None):
        if evs: evs[0].record(stream)
        layer.route(x, wr, bias, s, buf)
        if evs: evs[1].record(stream)
        layer.permute(x, s, buf)
        if evs: evs[2].record(stream)
        if buf.fused_gather:
            L.moe_grouped_gemm(x, w_gu, buf.H, buf.offsets, L.MOE_EPI_SWIGLU, a_rows=buf.src_token,
                               workspace=buf.ws_gemm1)
        else:
            L.moe_grouped_gemm(buf.x_perm, w_gu, buf.H, buf.offsets, L.MOE_EPI_SWIGLU, workspace=buf.ws_gemm1)
        if evs: evs[3].record(stream)
        L.moe_grouped_gemm(buf.H, w_down, buf.Y, buf.offsets, L.MOE_EPI_NONE, workspace=buf.ws_gemm2)
        if evs: evs[4].record(stream)
        layer.combine(s, buf)
        if evs: evs[5].record(stream)

    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    # timed: each step starts with cold caches (the flush runs before the step's first event)
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        step(ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    parts = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(len(STAGES))] for i in range(args.steps)])
    step_ms = np.array([ev[i][0].elapsed_time(ev[i][-1]) for i in range(args.steps)])
    pm = np.median(parts, axis=0)   # per-stage medians (ms)
    ms = float(np.median(step_ms))
    # the same steps back to back with no flush (caches warm from the step before), for reference
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(args.steps):
        step()
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / args.steps
    graph_ms = time_graph(step, args.steps, flush)

    counts = np.diff(buf.offsets.cpu().numpy())[:w.E]
    flops = useful_flops(w, counts)
    rows = w.T * w.k + (w.T if w.shared_f else 0)
    g1_flops = 2.0 * rows * w.d * 2 * w.f
    g1_bytes = gemm1_bytes(w, counts, fused)
    g1_ms = pm[2]
    g1_tflops = g1_flops / (g1_ms * 1e-3) / 1e12
    g1_gbs = g1_bytes / (g1_ms * 1e-3) / 1e9
    t_hbm, t_mfma = g1_bytes / (HBM_PEAK_GBS * 1e9), g1_flops / (BF16_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(g1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(g1_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(g1_tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(g1_tflops / BF16_PEAK_TFLOPS, 4)}
    roof["traffic"] = pmc_traffic(w.name) if fused else None
    roof.update({"kernel": "moe_grouped_gemm gate/up+SwiGLU (schedule + main kernel)",
                 "algorithmic_bytes": g1_bytes, "algorithmic_flops": g1_flops, "ms": round(g1_ms, 4),
                 "tflops": round(g1_tflops, 1), "gbs": round(g1_gbs, 1),
                 "mfma_frac": round(g1_tflops / BF16_PEAK_TFLOPS, 4)})
    route_bytes = w.T * w.d * 2 + w.E * w.d * 2 + w.T * w.k * 8
    perm_bytes = w.T * w.k * 12 + (0 if fused else (w.T * w.d * 2 + rows * w.d * 2))
    comb_bytes = w.T * w.k * w.d * 2 + w.T * w.k * 8 + w.T * w.d * 2 + (w.T * w.d * 2 if w.shared_f else 0)
    gemm_ms = pm[2] + pm[3]
    res = {
        "metric": ("MoE layer grouped-GEMM TFLOPS (useful FLOPs) + tokens/s, DSv3-shaped bf16" if w.name == "dsv3"
                   else f"MoE layer grouped-GEMM TFLOPS (useful FLOPs) + tokens/s, {w.name} bf16"),
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded hash-table normal inputs, Zipf/linear expert-bias skew; random-init weights)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "f": w.f, "E": w.E, "k": w.k, "score": w.score,
                   "shared_f": w.shared_f, "gather": "fused into GEMM 1" if fused else "materialised x_perm",
                   "groups_nonempty": int(np.count_nonzero(counts)), "group_max": int(counts.max()),
                   "group_min": int(counts.min()), "groups_empty": int((counts == 0).sum())},
        "timing": ("median over the timed steps of HIP events on the launching stream; every timed step "
                   f"starts after a {FLUSH_BYTES >> 20} MiB read of a scratch buffer outside the events"),
        "step_ms": spread(step_ms),
        "wall_ms_per_step_incl_flush": round(wall_ms, 4),
        "graph_ms_per_step": spread(graph_ms),
        "warm_ms_per_step": round(warm_ms, 4),
        "tokens_per_s": round(w.T / (ms * 1e-3), 1),
        "gemm_tflops": round(flops / (gemm_ms * 1e-3) / 1e12, 2),
        "gemm_mfma_frac": round(flops / (gemm_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "stage_ms": {n: spread(parts[:, j]) for j, n in enumerate(STAGES)},
        "stage_gbs": {"route": round(route_bytes / (pm[0] * 1e-3) / 1e9, 1),
                      "permute": round(perm_bytes / (pm[1] * 1e-3) / 1e9, 1),
                      "combine": round(comb_bytes / (pm[4] * 1e-3) / 1e9, 1)},
        "stage_hbm_frac": {"route": round(route_bytes / (pm[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "combine": round(comb_bytes / (pm[4] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": roof,
        "cpu_baseline": None,
    }
    # The step fuses the gather into GEMM 1, so its permute moves only indices. The dispatch
    # with the gather written out (histogram, offsets, permutation and x_perm [T*k, d]: x read
    # once, each token row written to its k rows) is timed here on its own, outside the step,
    # on the step's routing and with a flush before each repetition, so the dispatch's HBM
    # rate is measured on real data movement. The shared expert reads x directly, so no
    # shared rows are copied here.
    gs = layer.LayerShape(T=w.T, d=w.d, f=w.f, E=w.E, k=w.k, shared=False, score=s.score)
    gbuf = layer.LayerBuffers(gs, dev, fused_gather=False)
    gbuf.topk_idx.copy_(buf.topk_idx)    # the step's routing
    for _ in range(2):
        layer.permute(x, gs, gbuf)
    reps = max(5, min(args.steps, 20))
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in pev:
        flush()
        e0.record(stream)
        layer.permute(x, gs, gbuf)
        e1.record(stream)
    torch.cuda.synchronize()
    pg = [e0.elapsed_time(e1) for e0, e1 in pev]
    pg_ms = float(np.median(pg))
    pg_bytes = w.T * w.d * 2 + w.T * w.k * w.d * 2 + w.T * w.k * 12
    tk = w.T * w.k
    same = bool(torch.equal(gbuf.src_token, buf.src_token[:tk]) and torch.equal(gbuf.offsets, buf.offsets[:w.E + 1]))
    res["permute_materialised"] = {"ms": spread(pg), "gbs": round(pg_bytes / (pg_ms * 1e-3) / 1e9, 1),
                                   "hbm_frac": round(pg_bytes / (pg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                   "bytes": pg_bytes, "indices_match_step": same}
    del gbuf
    if args.calibrate_copy:
        calibrate_copy(dev)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, w_gu, w_down)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
