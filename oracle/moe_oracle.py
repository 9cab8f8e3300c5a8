"""Oracle: a plain, slow, obviously correct CPU model of one dropless MoE layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP library or its Python binding.

Everything is numpy, accumulated in float64. Storage roundings of the GPU path are
mirrored explicitly at the tensor boundaries where the GPU materialises a tensor
(`rnd` = round-to-nearest-even to bfloat16, or to float32 for the fp32 workload), so that
the comparison measures kernel error rather than the difference between a bf16 pipeline
and an infinitely precise one. Passing `rnd=None` gives the pure fp64 variant.

Sources, cited by page and section (the pages describe the method in words only; they
print no equation, listing or worked example):
  [Blog]    "Accelerating Dropless MoE Training in JAX with NVIDIA Transformer Engine",
            Chinese rendering on zhiding.cn.
  [Card]    the knowledge card summarising the same blog (ai.cheesepanini.fun).
  [Reading] the paper-daily deep reading of arXiv 2603.07685.
  [OCP-MX]  OCP Microscaling Formats (MX) Specification v1.0, for what "MXFP8" means.

Readings where the pages are silent are marked READING and listed with the design notes.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64

# --------------------------------------------------------------------------------------
# storage roundings
# --------------------------------------------------------------------------------------

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range: the spacing of
    values in [2**(e-1), 2**e) is 2**(e-8), down to the subnormal spacing 2**-133.
    The rounding is done once, directly from float64 (no detour through float32).
    """
    a = np.asarray(a, dtype=F64)
    _, e = np.frexp(a)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(a, -q)), q)
    big = np.abs(r) > BF16_MAX
    if np.any(big):
        r = np.where(big, np.copysign(np.inf, a), r)
    return r


def round_f32(a) -> np.ndarray:
    """Round float64 values to the nearest float32 (ties to even), returned as float64."""
    return np.asarray(a, dtype=F64).astype(np.float32).astype(F64)


def _identity(a):
    return np.asarray(a, dtype=F64)


def _rounder(rnd):
    return _identity if rnd is None else rnd


# --------------------------------------------------------------------------------------
# route  ([Blog] "Optimisation 2": a fused router kernel assigns each token its experts;
#         [Blog] opening: a learnable router picks the top-K experts of each token)
# --------------------------------------------------------------------------------------

def router_logits(x, w_router) -> np.ndarray:
    """L[t, e] = sum_i x[t, i] * w_router[e, i], exact in float64 for bf16 inputs.

    READING: the router is a bias-free linear projection; w_router is stored [E, d].
    """
    return np.asarray(x, F64) @ np.asarray(w_router, F64).T


def router_keys(x, w_router, bias=None) -> np.ndarray:
    """Selection keys in float32: kappa = fl32(fl32(L) + b).

    READING: the per-expert bias is added to the logit; the sum is the key that both
    selects experts and feeds the score function. Where floating point decides the
    selection, the decision is taken in float32, the precision of the GPU's logits.
    """
    k = round_f32(router_logits(x, w_router))
    if bias is not None:
        k = round_f32(k + np.asarray(bias, F64)[None, :])
    return k.astype(np.float32)


def select_topk(keys, k: int) -> np.ndarray:
    """The k experts with the largest keys, largest first; equal keys go to the lower id.

    READING: the pages do not fix a tie-break or an output order; this one makes the
    answer unique. A stable ascending sort of the negated keys keeps equal keys in
    expert-id order.
    """
    keys = np.asarray(keys)
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def topk_weights(keys, topk_idx, score: str) -> np.ndarray:
    """Routing weights of the selected experts, normalised to sum to one per token.

    softmax: exp(kappa_j) / sum over the k selected exp(kappa_j'); this equals a softmax
             over all experts renormalised over the selected ones.
    sigmoid: s_j = 1 / (1 + exp(-kappa_j)), w_j = s_j / sum_j' s_j'.
    READING: every workload normalises its top-k weights; no routed scaling factor.
    """
    kk = np.take_along_axis(np.asarray(keys, F64), np.asarray(topk_idx, np.int64), axis=1)
    if score == "softmax":
        z = np.exp(kk - kk[:, :1])
    elif score == "sigmoid":
        z = 1.0 / (1.0 + np.exp(-kk))
    else:
        raise ValueError(score)
    return z / z.sum(axis=1, keepdims=True)


def route(x, w_router, bias, k: int, score: str):
    """Full routing: returns (topk_idx int32 [T,k], topk_w float64 [T,k], keys float32 [T,E])."""
    keys = router_keys(x, w_router, bias)
    idx = select_topk(keys, k)
    return idx, topk_weights(keys, idx, score), keys


def topk_weights_backward(keys, topk_idx, d_topk_w, score: str) -> np.ndarray:
    """Gradient with respect to the keys [T, E] of a loss whose gradient with respect to the
    normalised routing weights is d_topk_w [T, k]. The selection is piecewise constant in the
    keys, so only the selected experts receive gradient ([Blog] opening section: the router
    picks the top-K experts; READING: the router's own backward is the derivative of the
    weight formula of topk_weights with the selection held fixed).

    softmax: w = softmax over the selected keys, so d kappa_j = w_j (g_j - sum_i w_i g_i).
    sigmoid: w_j = s_j / S with S = sum_i s_i, so dL/ds_j = (g_j - sum_i w_i g_i) / S and
             d kappa_j = dL/ds_j * s_j (1 - s_j).
    """
    keys = np.asarray(keys, F64)
    idx = np.asarray(topk_idx, np.int64)
    g = np.asarray(d_topk_w, F64)
    kk = np.take_along_axis(keys, idx, axis=1)
    if score == "softmax":
        z = np.exp(kk - kk[:, :1])
        w = z / z.sum(axis=1, keepdims=True)
        dk = w * (g - (w * g).sum(axis=1, keepdims=True))
    elif score == "sigmoid":
        sg = 1.0 / (1.0 + np.exp(-kk))
        S = sg.sum(axis=1, keepdims=True)
        w = sg / S
        dk = (g - (w * g).sum(axis=1, keepdims=True)) / S * sg * (1.0 - sg)
    else:
        raise ValueError(score)
    out = np.zeros_like(keys)
    np.put_along_axis(out, idx, dk, axis=1)
    return out


def router_backward(x, w_router, d_keys):
    """The keys are x W_r^T + b, so with G = d_keys [T, E]: dW_r = G^T x [E, d],
    dx = G W_r [T, d] (the router's share of the input gradient), d_bias = column sums [E]."""
    G = np.asarray(d_keys, F64)
    return G.T @ np.asarray(x, F64), G @ np.asarray(w_router, F64), G.sum(axis=0)


# --------------------------------------------------------------------------------------
# dispatch: counts, offsets, permutation, gather
#   ([Blog] "Optimisation 2": dispatch reorders tokens locally so each expert's tokens
#    are contiguous; combine restores the original order. [Blog] "Optimisation 1" and
#    "Optimisations dropless MoE needs": group sizes stay on the device.)
# --------------------------------------------------------------------------------------

def permutation(topk_idx, E: int, shared_rows: int = 0):
    """Stable counting sort of the (token, slot) pairs by expert.

    Returns offsets int32 [E+1] (or [E+2] with a shared group), row_of int32 [T,k] and
    src_token int32 [T*k (+ shared_rows)]. Rows of one expert are contiguous and in
    ascending token order (READING: any order is valid; this one is reproducible). When
    shared_rows = T, group E holds every token in order (the always-on shared expert).
    """
    idx = np.asarray(topk_idx, np.int64)
    T, k = idx.shape
    e_flat = idx.reshape(-1)
    t_flat = np.repeat(np.arange(T, dtype=np.int64), k)
    order = np.lexsort((t_flat, e_flat))          # primary key expert, then token
    src = t_flat[order]
    row_of = np.empty(T * k, dtype=np.int64)
    row_of[order] = np.arange(T * k)
    counts = np.bincount(e_flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    if shared_rows:
        offsets = np.concatenate([offsets, [offsets[-1] + shared_rows]])
        src = np.concatenate([src, np.arange(shared_rows)])
    return offsets.astype(np.int32), row_of.reshape(T, k).astype(np.int32), src.astype(np.int32)


def gather_rows(x, src_token) -> np.ndarray:
    """x_perm[r] = x[src_token[r]]: a pure copy."""
    return np.asarray(x)[np.asarray(src_token, np.int64)]


# --------------------------------------------------------------------------------------
# experts: SwiGLU MLP per group  ([Blog] Figure 3 paragraph: the grouped MLP runs two
#   grouped GEMMs over the variable-length groups; [Blog] "Optimisation 1": one call
#   covers every expert at its actual token count)
# --------------------------------------------------------------------------------------

def silu(z):
    z = np.asarray(z, F64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def silu_grad(z):
    """d/dz [z * sigma(z)] = sigma(z) * (1 + z * (1 - sigma(z)))."""
    z = np.asarray(z, F64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def expert_gate_up(X, w_gu_e):
    """G = X W_gate^T, U = X W_up^T; w_gu_e is [2f, d] with gate rows first (READING)."""
    f = w_gu_e.shape[0] // 2
    X = np.asarray(X, F64)
    W = np.asarray(w_gu_e, F64)
    return X @ W[:f].T, X @ W[f:].T


def expert_forward(X, w_gu_e, w_down_e, rnd=None, mx=False, return_gu=False, mx4=False):
    """H = rnd(silu(G) * U), Y = rnd(H W_down^T); returns (H, Y) (and (G, U) unrounded).

    w_down_e is [d, f]. With `mx` (MXFP8) or `mx4` (MXFP4), each GEMM operand first passes
    through that format's rowwise quantiser along its contraction axis (X and W_gu along d,
    H and W_down along f).
    """
    r = _rounder(rnd)
    q = mx4_q_rows if mx4 else mx_q_rows
    mx = mx or mx4
    if mx:
        X, w_gu_e, w_down_e = q(X), q(w_gu_e), q(w_down_e)
    G, U = expert_gate_up(X, w_gu_e)
    H = r(silu(G) * U)
    Hq = q(H) if mx else H
    Y = r(Hq @ np.asarray(w_down_e, F64).T)
    if return_gu:
        return H, Y, (G, U)
    return H, Y


def grouped_gemm(A, W, offsets, a_row_index=None, rnd=None):
    """Plain grouped GEMM: C[o_g:o_{g+1}] = A[rows of g] W[g]^T for each group g.

    A is [rows, K], W is [G, N, K]; with a_row_index, row r of the output reads A row
    a_row_index[r]. Empty groups produce nothing.
    """
    r = _rounder(rnd)
    offsets = np.asarray(offsets, np.int64)
    G = len(offsets) - 1
    M = int(offsets[-1])
    C = np.zeros((M, W.shape[1]), dtype=F64)
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi == lo:
            continue
        rows = np.arange(lo, hi) if a_row_index is None else np.asarray(a_row_index, np.int64)[lo:hi]
        C[lo:hi] = np.asarray(A, F64)[rows] @ np.asarray(W[g], F64).T
    return r(C)


def grouped_swiglu(A, W_gu, offsets, a_row_index=None, rnd=None):
    """Grouped GEMM 1 with the SwiGLU epilogue: H rows of group g = rnd(silu(G) * U)."""
    r = _rounder(rnd)
    offsets = np.asarray(offsets, np.int64)
    G = len(offsets) - 1
    f = W_gu.shape[1] // 2
    H = np.zeros((int(offsets[-1]), f), dtype=F64)
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi == lo:
            continue
        rows = np.arange(lo, hi) if a_row_index is None else np.asarray(a_row_index, np.int64)[lo:hi]
        Gm, Um = expert_gate_up(np.asarray(A, F64)[rows], W_gu[g])
        H[lo:hi] = silu(Gm) * Um
    return r(H)


# --------------------------------------------------------------------------------------
# combine  ([Blog] "Optimisation 2": combine returns every expert output to its token's
#   original position and accumulates them)
# --------------------------------------------------------------------------------------

def combine(Y, topk_w, row_of, y_shared=None, rnd=None):
    """out[t] = rnd(sum_j w[t,j] * Y[row_of[t,j]] + y_shared[t]), summed in float64.

    READING: the shared expert is always on with weight one and joins the same sum
    before the single output rounding.
    """
    r = _rounder(rnd)
    Y = np.asarray(Y, F64)
    w = np.asarray(topk_w, F64)
    ro = np.asarray(row_of, np.int64)
    acc = np.zeros((ro.shape[0], Y.shape[1]), dtype=F64)
    for j in range(ro.shape[1]):
        acc += w[:, j:j + 1] * Y[ro[:, j]]
    if y_shared is not None:
        acc += np.asarray(y_shared, F64)
    return r(acc)


# --------------------------------------------------------------------------------------
# whole forward
# --------------------------------------------------------------------------------------

def layer_forward(x, w_router, bias, k, score, w_gu, w_down, E, shared=False, rnd=None,
                  topk=None, mx=False, mx4=False):
    """One dropless MoE layer forward: route -> permute -> grouped SwiGLU MLP -> combine.

    w_gu(e) / w_down(e) return expert e's [2f, d] / [d, f] weights (e = E is the shared
    expert when `shared`). `topk` = (idx, w) skips the routing step. Returns a dict of
    every intermediate the GPU path materialises.
    [Reading] "Method overview": route, dispatch, compute, combine.
    [Blog] "Dropless vs capacity-based MoE": no token is dropped and nothing is padded.
    """
    x = np.asarray(x, F64)
    T = x.shape[0]
    if topk is None:
        idx, w, keys = route(x, w_router, bias, k, score)
    else:
        (idx, w), keys = topk, None
    offsets, row_of, src = permutation(idx, E, T if shared else 0)
    xp = gather_rows(x, src)
    f = None
    H_parts, Y_parts = [], []
    n_groups = E + (1 if shared else 0)
    for g in range(n_groups):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi == lo:
            continue
        H, Y = expert_forward(xp[lo:hi], w_gu(g), w_down(g), rnd, mx=mx, mx4=mx4)
        H_parts.append((lo, H))
        Y_parts.append((lo, Y))
        f = H.shape[1]
    M = int(offsets[-1])
    Hm = np.zeros((M, f if f else 0), F64)
    Ym = np.zeros((M, x.shape[1]), F64)
    for lo, H in H_parts:
        Hm[lo:lo + H.shape[0]] = H
    for lo, Y in Y_parts:
        Ym[lo:lo + Y.shape[0]] = Y
    y_shared = Ym[T * k:] if shared else None
    out = combine(Ym[:T * k], w, row_of, y_shared, rnd)
    return dict(topk_idx=idx, topk_w=w, keys=keys, offsets=offsets, row_of=row_of,
                src_token=src, x_perm=xp, H=Hm, Y=Ym, out=out)


def layer_forward_per_token(x, w_router, bias, k, score, w_gu, w_down, E, shared=False):
    """Brute force: out[t] = sum_j w[t,j] * MLP_{S[t,j]}(x[t]) (+ shared MLP), pure fp64,
    token by token with no permutation at all."""
    x = np.asarray(x, F64)
    idx, w, _ = route(x, w_router, bias, k, score)
    out = np.zeros_like(x)
    for t in range(x.shape[0]):
        for j in range(k):
            _, y = expert_forward(x[t:t + 1], w_gu(int(idx[t, j])), w_down(int(idx[t, j])))
            out[t] += w[t, j] * y[0]
        if shared:
            _, y = expert_forward(x[t:t + 1], w_gu(E), w_down(E))
            out[t] += y[0]
    return out


# --------------------------------------------------------------------------------------
# MXFP8  ([Blog] "Optimisations dropless MoE needs": group-aware MXFP8 quantisation and an
#   MXFP8 grouped GEMM; [Reading] contribution 3: MoE low precision needs group
#   quantisation. [OCP-MX] section 5 and 6 define the block format used here.)
# --------------------------------------------------------------------------------------

E4M3_MAX = 448.0
MX_BLOCK = 32


def e4m3_round(v) -> np.ndarray:
    """Round float64 values to the nearest OCP E4M3 value (ties to even), saturating.

    E4M3 ([OCP-MX] FP8 E4M3): exponent bias 7, 3 mantissa bits, normals down to 2**-6,
    subnormal spacing 2**-9, largest finite 448, no infinities. Magnitudes above 448
    saturate to 448 (READING: the MX conversion clamps to the largest normal).
    """
    v = np.asarray(v, F64)
    a = np.abs(v)
    _, e = np.frexp(a)
    q = np.maximum(e - 4, -9)
    r = np.ldexp(np.rint(np.ldexp(a, -q)), q)
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, v)


def e4m3_encode(r) -> np.ndarray:
    """Byte code of values already on the E4M3 grid (sign bit kept, also for zero)."""
    r = np.asarray(r, F64)
    a = np.abs(r)
    sign = np.signbit(r).astype(np.uint16) << 7
    _, e = np.frexp(a)
    exp_unb = e - 1                                 # a in [2**exp_unb, 2**(exp_unb+1))
    normal = a >= 2.0 ** -6
    ef = np.where(normal, exp_unb + 7, 0)
    mant = np.where(normal, np.ldexp(a, -exp_unb) - 1.0, np.ldexp(a, 9)) * np.where(normal, 8.0, 1.0)
    mant = np.rint(mant).astype(np.int64)
    code = sign | (ef.astype(np.uint16) << 3) | mant.astype(np.uint16)
    return code.astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    c = np.asarray(code, np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(ef == 0, np.ldexp(m.astype(F64), -9), np.ldexp(1.0 + m / 8.0, ef - 7))
    mag = np.where((ef == 15) & (m == 7), np.nan, mag)
    return s * mag


def mx_scale_byte(amax) -> np.ndarray:
    """E8M0 shared-scale byte of a block from its largest magnitude.

    [OCP-MX] section 6.3: shared exponent = floor(log2(amax)) - emax_elem, emax_elem = 8
    for E4M3; the byte is that exponent plus 127, clamped to the representable 0..254.
    An all-zero block gets byte 0.
    """
    amax = np.asarray(amax, F64)
    _, e = np.frexp(amax)                  # amax = m * 2**e, m in [0.5, 1) -> floor(log2) = e - 1
    b = np.clip(e - 1 - 8 + 127, 0, 254)
    return np.where(amax > 0, b, 0).astype(np.uint8)


def mx_quantize_blocks(blocks):
    """Quantise blocks [..., n<=32] (padding elements, if any, must be zero).

    Returns (codes uint8 [..., n], scale bytes uint8 [...], dequantised float64 [..., n]).
    """
    blocks = np.asarray(blocks, F64)
    amax = np.max(np.abs(blocks), axis=-1)
    sb = mx_scale_byte(amax)
    X = np.ldexp(1.0, sb.astype(np.int64) - 127)
    r = e4m3_round(blocks / X[..., None])
    return e4m3_encode(r), sb, r * X[..., None]


def mx_quantize_rowwise(a):
    """Blocks of 32 consecutive elements along each row (a is [rows, cols], cols % 32 == 0).

    Returns codes [rows, cols], scales [rows, cols/32], dequantised [rows, cols].
    """
    a = np.asarray(a, F64)
    R, C = a.shape
    assert C % MX_BLOCK == 0
    codes, sb, dq = mx_quantize_blocks(a.reshape(R, C // MX_BLOCK, MX_BLOCK))
    return codes.reshape(R, C), sb, dq.reshape(R, C)


def mx_quantize_colwise_grouped(a, offsets):
    """Blocks of 32 consecutive ROWS inside each group, per column (the wgrad operand).

    [Blog] "Optimisations dropless MoE needs": the quantiser is group-aware. READING:
    a block never straddles a group boundary; a group's last block may be partial and its
    missing rows count as zeros. Returns (codes [rows, cols], scales list per group of
    [ceil(m_g/32), cols], dequantised [rows, cols]).
    """
    a = np.asarray(a, F64)
    offsets = np.asarray(offsets, np.int64)
    codes = np.zeros(a.shape, np.uint8)
    dq = np.zeros(a.shape, F64)
    scales = []
    for g in range(len(offsets) - 1):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        m = hi - lo
        nb = (m + MX_BLOCK - 1) // MX_BLOCK
        if nb == 0:
            scales.append(np.zeros((0, a.shape[1]), np.uint8))
            continue
        pad = np.zeros((nb * MX_BLOCK, a.shape[1]), F64)
        pad[:m] = a[lo:hi]
        blk = pad.reshape(nb, MX_BLOCK, a.shape[1]).transpose(0, 2, 1)   # [nb, cols, 32]
        c, sb, d = mx_quantize_blocks(blk)
        codes[lo:hi] = c.transpose(0, 2, 1).reshape(nb * MX_BLOCK, -1)[:m]
        dq[lo:hi] = d.transpose(0, 2, 1).reshape(nb * MX_BLOCK, -1)[:m]
        scales.append(sb)
    return codes, scales, dq


def mx_q_rows(a):
    """Dequantised value of a after rowwise MX quantisation (the operator Q along rows)."""
    return mx_quantize_rowwise(a)[2]


# --------------------------------------------------------------------------------------
# MXFP4  ([Blog] "JAX plus Transformer Engine MoE training performance": a 4-bit block-scaled
#   format is the planned next precision; [Reading] contribution 3: FP8/FP4 recipes.
#   [OCP-MX] defines MXFP4 as E2M1 elements sharing one E8M0 scale per block of 32.)
# --------------------------------------------------------------------------------------

E2M1_MAX = 6.0


def e2m1_round(v) -> np.ndarray:
    """Round float64 values to the nearest OCP E2M1 value (ties to even), saturating.

    E2M1 ([OCP-MX] FP4 E2M1): exponent bias 1, 1 mantissa bit, normals 1, 1.5, 2, 3, 4, 6
    (exponent 0..2), subnormal 0.5, largest finite 6, no infinities or NaN. The spacing is
    2**(floor(log2|v|) - 1) for |v| >= 1 and 0.5 below; magnitudes above 6 saturate to 6
    (READING: the MX conversion clamps to the largest normal, as for E4M3).
    """
    v = np.asarray(v, F64)
    a = np.abs(v)
    _, e = np.frexp(a)                      # a = m 2**e, m in [0.5, 1): floor(log2 a) = e - 1
    q = np.maximum(e - 2, -1)
    r = np.ldexp(np.rint(np.ldexp(a, -q)), q)
    r = np.minimum(r, E2M1_MAX)
    return np.copysign(r, v)


def e2m1_encode(r) -> np.ndarray:
    """4-bit code of values already on the E2M1 grid: sign in bit 3, exponent field in bits
    2..1, mantissa in bit 0 (the sign bit kept, also for zero)."""
    r = np.asarray(r, F64)
    a = np.abs(r)
    sign = np.signbit(r).astype(np.int64) << 3
    _, e = np.frexp(a)
    normal = a >= 1.0
    ef = np.where(normal, e, 0)             # a in [2**(e-1), 2**e): exponent field (e - 1) + 1
    mant = np.where(normal, np.ldexp(a, 1 - e) * 2.0 - 2.0, a * 2.0)
    return (sign | (ef.astype(np.int64) << 1) | np.rint(mant).astype(np.int64)).astype(np.uint8)


def e2m1_decode(code) -> np.ndarray:
    c = np.asarray(code, np.int64)
    s = np.where(c & 0x8, -1.0, 1.0)
    ef = (c >> 1) & 0x3
    m = c & 1
    mag = np.where(ef == 0, 0.5 * m, np.ldexp(1.0 + m / 2.0, ef - 1))
    return s * mag


def mx4_scale_byte(amax) -> np.ndarray:
    """E8M0 shared-scale byte of an MXFP4 block: [OCP-MX] section 6.3 with emax_elem = 2 for
    E2M1 (largest normal 6 = 1.5 * 2**2); an all-zero block gets byte 0."""
    amax = np.asarray(amax, F64)
    _, e = np.frexp(amax)
    b = np.clip(e - 1 - 2 + 127, 0, 254)
    return np.where(amax > 0, b, 0).astype(np.uint8)


def mx4_quantize_blocks(blocks):
    """Quantise blocks [..., n<=32] to MXFP4 (padding elements, if any, must be zero).

    Returns (4-bit codes uint8 [..., n], scale bytes uint8 [...], dequantised float64 [..., n]).
    """
    blocks = np.asarray(blocks, F64)
    amax = np.max(np.abs(blocks), axis=-1)
    sb = mx4_scale_byte(amax)
    X = np.ldexp(1.0, sb.astype(np.int64) - 127)
    r = e2m1_round(blocks / X[..., None])
    return e2m1_encode(r), sb, r * X[..., None]


def mx4_quantize_rowwise(a):
    """MXFP4 blocks of 32 consecutive elements along each row (cols % 32 == 0): codes [rows,
    cols] (one 4-bit code per element), scales [rows, cols/32], dequantised [rows, cols]."""
    a = np.asarray(a, F64)
    R, C = a.shape
    assert C % MX_BLOCK == 0
    codes, sb, dq = mx4_quantize_blocks(a.reshape(R, C // MX_BLOCK, MX_BLOCK))
    return codes.reshape(R, C), sb, dq.reshape(R, C)


def mx4_q_rows(a):
    """Dequantised value of a after row-wise MXFP4 quantisation."""
    return mx4_quantize_rowwise(a)[2]


# --------------------------------------------------------------------------------------
# backward (the expert/permute/combine part; the router's own backward is not included)
# --------------------------------------------------------------------------------------

def combine_backward(d_out, Y, topk_w, row_of, rnd=None):
    """Transpose of combine: dY[row_of[t,j]] = w[t,j] d_out[t]; dw[t,j] = <d_out[t], Y row>."""
    r = _rounder(rnd)
    d_out = np.asarray(d_out, F64)
    ro = np.asarray(row_of, np.int64)
    T, k = ro.shape
    dY = np.zeros((T * k, d_out.shape[1]), F64)
    dw = np.zeros((T, k), F64)
    for j in range(k):
        dY[ro[:, j]] = np.asarray(topk_w, F64)[:, j:j + 1] * d_out
        dw[:, j] = np.sum(d_out * np.asarray(Y, F64)[ro[:, j]], axis=1)
    return r(dY), dw


def permute_backward(dX_perm, row_of, dx_shared=None, rnd=None):
    """Transpose of the gather: dx[t] = sum_j dX_perm[row_of[t,j]] (+ dx_shared[t])."""
    r = _rounder(rnd)
    dX_perm = np.asarray(dX_perm, F64)
    ro = np.asarray(row_of, np.int64)
    acc = np.zeros((ro.shape[0], dX_perm.shape[1]), F64)
    for j in range(ro.shape[1]):
        acc += dX_perm[ro[:, j]]
    if dx_shared is not None:
        acc += np.asarray(dx_shared, F64)
    return r(acc)


def expert_backward(X, w_gu_e, w_down_e, dY, rnd=None, mx=False):
    """Backward of one SwiGLU expert on its rows X [m, d] given dY [m, d].

    Returns dict(dX [m,d], dW_gu [2f,d], dW_down [d,f], dH, dG, dU and the forward's H, G, U).
    The forward is recomputed here exactly as `expert_forward` computes it. READING: the
    forward stores G and U rounded to storage (Gs, Us) and the SwiGLU backward uses those:
    dG = rnd(dH * Us * silu'(Gs)), dU = rnd(dH * silu(Gs)).
    With `mx`, every GEMM operand is first MX-quantised along that GEMM's contraction
    axis: rowwise blocks for the data-gradient GEMMs (dY along d with W_down's columns
    along d; dGU along 2f with W_gu's columns along 2f), and 32-row blocks inside the group
    for the weight-gradient GEMMs, whose contraction runs over the group's tokens.
    """
    r = _rounder(rnd)
    X = np.asarray(X, F64)
    Wgu = np.asarray(w_gu_e, F64)
    Wd = np.asarray(w_down_e, F64)
    dY = np.asarray(dY, F64)
    m = X.shape[0]
    H, _, (G, U) = expert_forward(X, Wgu, Wd, rnd, mx=mx, return_gu=True)
    Gs, Us = r(G), r(U)
    off = np.array([0, m])
    if mx:
        dH = r(mx_q_rows(dY) @ mx_q_rows(Wd.T).T)
        dWd = r(mx_quantize_colwise_grouped(dY, off)[2].T @ mx_quantize_colwise_grouped(H, off)[2])
    else:
        dH = r(dY @ Wd)
        dWd = r(dY.T @ H)
    dG = r(dH * Us * silu_grad(Gs))
    dU = r(dH * silu(Gs))
    dGU = np.concatenate([dG, dU], axis=1)
    if mx:
        dX = r(mx_q_rows(dGU) @ mx_q_rows(Wgu.T).T)
        dWgu = r(mx_quantize_colwise_grouped(dGU, off)[2].T @ mx_quantize_colwise_grouped(X, off)[2])
    else:
        dX = r(dGU @ Wgu)
        dWgu = r(dGU.T @ X)
    return dict(dX=dX, dW_gu=dWgu, dW_down=dWd, dH=dH, dG=dG, dU=dU, H=H, G=G, U=U)


def layer_backward(fwd, d_out, w_gu, w_down, E, shared=False, rnd=None, mx=False, router=None):
    """Backward of the expert, permute and combine steps of `layer_forward`'s result.

    Returns dict(dx [T,d], dY [T*k,d] (routed rows), dw [T,k], dW_gu {g: [2f,d]},
    dW_down {g: [d,f]}, dX_perm [rows,d]). An empty group's weight gradients are zeros.

    router = (x, w_router, score) adds the router's backward ([Blog] opening section: the
    router is trained with the layer, so the loss reaches the keys through the routing
    weights): d_keys [T,E], dW_router [E,d], d_bias [E], and the layer input's gradient
    becomes the expert path's (as stored) plus the router's share, rounded once.
    """
    r = _rounder(rnd)
    T, k = fwd["row_of"].shape
    offsets = np.asarray(fwd["offsets"], np.int64)
    Y = fwd["Y"]
    dY_r, dw = combine_backward(d_out, Y[:T * k], fwd["topk_w"], fwd["row_of"], rnd)
    dY = np.concatenate([dY_r, r(np.asarray(d_out, F64))], axis=0) if shared else dY_r
    dXp = np.zeros_like(fwd["x_perm"], dtype=F64)
    dWgu, dWd = {}, {}
    for g in range(E + (1 if shared else 0)):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        Wgu, Wd = w_gu(g), w_down(g)
        if hi == lo:
            dWgu[g] = np.zeros(Wgu.shape, F64)
            dWd[g] = np.zeros(Wd.shape, F64)
            continue
        res = expert_backward(fwd["x_perm"][lo:hi], Wgu, Wd, dY[lo:hi], rnd, mx)
        dXp[lo:hi] = res["dX"]
        dWgu[g], dWd[g] = res["dW_gu"], res["dW_down"]
    dx = permute_backward(dXp[:T * k], fwd["row_of"], dXp[T * k:] if shared else None, rnd)
    out = dict(dx=dx, dY=dY, dw=dw, dW_gu=dWgu, dW_down=dWd, dX_perm=dXp)
    if router is not None:
        x, w_router, score = router
        d_keys = topk_weights_backward(fwd["keys"], fwd["topk_idx"], dw, score)
        dWr, dx_r, db = router_backward(x, w_router, d_keys)
        out.update(dx=r(dx + dx_r), d_keys=d_keys, dW_router=dWr, d_bias=db)
    return out
