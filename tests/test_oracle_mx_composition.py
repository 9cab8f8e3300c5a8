"""CPU pin of the oracle's MXFP8 composition: which operand of which GEMM is quantised, and
along which axis.

[Blog] "Optimisations dropless MoE needs": the expert GEMMs run in MXFP8 with group-aware
quantisation; [OCP-MX]: a block is 32 consecutive elements sharing one E8M0 scale. A block
only makes sense along the axis a product contracts over, so every GEMM operand of the
training step is quantised along that GEMM's contraction axis: the forward and data-gradient
GEMMs along the rows' length (d, f or 2f), the weight-gradient GEMMs over the group's tokens,
in 32-row blocks that start at the group's first row, the last one possibly partial.

The brute force below rebuilds every element of Y, dH, dW_down, dX and dW_gu from explicit
blocks cut out of the operand vectors element by element, quantises each block on its own
with the pinned block quantiser, and sums the exact products with math.fsum. It shares no
matrix code with the oracle (no reshape of blocks, no transposed quantisation, no BLAS).
Each negative control recomputes one tensor with one operand quantised along the wrong axis
and must disagree with the oracle, so an oracle carrying that mistake would fail here.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import moe_oracle as O

BLK = 32


def q_block(vals):
    """Dequantised values of one block (fewer than 32 values: the missing ones are zero)."""
    blk = np.zeros((1, BLK))
    blk[0, :len(vals)] = vals
    return O.mx_quantize_blocks(blk)[2][0, :len(vals)]


def q_vec(vec):
    """A vector cut into consecutive 32-element blocks from its first element, each block
    quantised on its own (the last block may be partial)."""
    vec = np.asarray(vec, np.float64)
    out = np.empty_like(vec)
    for s in range(0, len(vec), BLK):
        out[s:s + BLK] = q_block(vec[s:s + BLK])
    return out


def dot(a, b):
    return math.fsum(float(x) * float(y) for x, y in zip(a, b))


def rnd(v):
    return float(O.round_bf16(np.float64(v)))


def silu(z):
    return z / (1.0 + math.exp(-z))


def silu_grad(z):
    s = 1.0 / (1.0 + math.exp(-z))
    return s * (1.0 + z * (1.0 - s))


class Case:
    """One expert's group of m tokens: X [m, d], W_gu [2f, d] (gate rows first), W_down [d, f],
    dY [m, d]; bf16-valued as the step stores them."""

    def __init__(self, m=37, d=64, f=64, seed=7):
        g = np.random.Generator(np.random.PCG64(seed))
        self.m, self.d, self.f = m, d, f
        self.X = O.round_bf16(g.standard_normal((m, d)))
        self.Wgu = O.round_bf16(g.standard_normal((2 * f, d)) * 0.02)
        self.Wd = O.round_bf16(g.standard_normal((d, f)) * 0.02)
        self.dY = O.round_bf16(g.standard_normal((m, d)))


def brute(c: Case, wrong: str = ""):
    """Every output of the MXFP8 expert forward and backward, element by element.

    `wrong` names one operand to quantise along the wrong axis (negative controls):
      "G:Wgu"    W_gu along 2f (its rows' length is d, the contraction of G and U)
      "Y:Wd"     W_down along d for Y (Y contracts over f)
      "Y:H"      H in 32-row blocks for Y (Y contracts over f)
      "dH:Wd"    W_down along f for dH (dH contracts over d)
      "dWd:dY"   dY along d for dW_down (dW_down contracts over the group's tokens)
      "dX:Wgu"   W_gu along d for dX (dX contracts over 2f)
      "dWgu:X"   X along d for dW_gu (dW_gu contracts over the group's tokens)
    """
    m, d, f = c.m, c.d, c.f
    # forward: G, U contract over d; X rows and W_gu rows (length d) blocked along d
    Xq = [q_vec(c.X[i]) for i in range(m)]
    if wrong == "G:Wgu":
        cols = [q_vec(c.Wgu[:, j]) for j in range(d)]          # blocks along 2f
        Wguq = [np.array([cols[j][r] for j in range(d)]) for r in range(2 * f)]
    else:
        Wguq = [q_vec(c.Wgu[r]) for r in range(2 * f)]
    G = np.array([[dot(Xq[i], Wguq[n]) for n in range(f)] for i in range(m)])
    U = np.array([[dot(Xq[i], Wguq[f + n]) for n in range(f)] for i in range(m)])
    H = np.array([[rnd(silu(G[i, n]) * U[i, n]) for n in range(f)] for i in range(m)])
    # Y contracts over f: H rows and W_down rows (length f) blocked along f
    if wrong == "Y:H":
        hc = [q_vec(H[:, n]) for n in range(f)]
        Hq = [np.array([hc[n][i] for n in range(f)]) for i in range(m)]
    else:
        Hq = [q_vec(H[i]) for i in range(m)]
    if wrong == "Y:Wd":
        wc = [q_vec(c.Wd[:, n]) for n in range(f)]
        Wdq = [np.array([wc[n][e] for n in range(f)]) for e in range(d)]
    else:
        Wdq = [q_vec(c.Wd[e]) for e in range(d)]
    Y = np.array([[rnd(dot(Hq[i], Wdq[e])) for e in range(d)] for i in range(m)])
    # dH contracts over d: dY rows blocked along d, W_down columns (length d) blocked along d
    dYq = [q_vec(c.dY[i]) for i in range(m)]
    if wrong == "dH:Wd":
        WdTq = [np.array([q_vec(c.Wd[e])[n] for e in range(d)]) for n in range(f)]
    else:
        WdTq = [q_vec(c.Wd[:, n]) for n in range(f)]
    dH = np.array([[rnd(dot(dYq[i], WdTq[n])) for n in range(f)] for i in range(m)])
    # dW_down[e, n] contracts over the group's tokens: dY and H columns in 32-row blocks
    if wrong == "dWd:dY":
        dYc = [np.array([dYq[i][e] for i in range(m)]) for e in range(d)]
    else:
        dYc = [q_vec(c.dY[:, e]) for e in range(d)]
    Hc = [q_vec(H[:, n]) for n in range(f)]
    dWd = np.array([[rnd(dot(dYc[e], Hc[n])) for n in range(f)] for e in range(d)])
    # SwiGLU backward on the stored (bf16) pre-activations
    dGU = np.zeros((m, 2 * f))
    for i in range(m):
        for n in range(f):
            gs, us = rnd(G[i, n]), rnd(U[i, n])
            dGU[i, n] = rnd(dH[i, n] * us * silu_grad(gs))
            dGU[i, f + n] = rnd(dH[i, n] * silu(gs))
    # dX contracts over 2f: dGU rows and W_gu columns (length 2f) blocked along 2f
    dGUq = [q_vec(dGU[i]) for i in range(m)]
    if wrong == "dX:Wgu":
        WguTq = [np.array([q_vec(c.Wgu[r])[j] for r in range(2 * f)]) for j in range(d)]
    else:
        WguTq = [q_vec(c.Wgu[:, j]) for j in range(d)]
    dX = np.array([[rnd(dot(dGUq[i], WguTq[j])) for j in range(d)] for i in range(m)])
    # dW_gu[r, j] contracts over the group's tokens: dGU and X columns in 32-row blocks
    dGUc = [q_vec(dGU[:, r]) for r in range(2 * f)]
    if wrong == "dWgu:X":
        Xc = [np.array([Xq[i][j] for i in range(m)]) for j in range(d)]
    else:
        Xc = [q_vec(c.X[:, j]) for j in range(d)]
    dWgu = np.array([[rnd(dot(dGUc[r], Xc[j])) for j in range(d)] for r in range(2 * f)])
    return dict(H=H, Y=Y, dH=dH, dW_down=dWd, dX=dX, dW_gu=dWgu)


def oracle(c: Case):
    res = O.expert_backward(c.X, c.Wgu, c.Wd, c.dY, rnd=O.round_bf16, mx=True)
    _, Y = O.expert_forward(c.X, c.Wgu, c.Wd, O.round_bf16, mx=True)
    res["Y"] = Y
    return res


@pytest.fixture(scope="module")
def case_and_oracle():
    c = Case()
    return c, oracle(c), brute(c)


@pytest.mark.parametrize("name", ["H", "Y", "dH", "dW_down", "dX", "dW_gu"])
def test_mx_composition_matches_blockwise_brute_force(case_and_oracle, name):
    """The group has 37 rows, so the weight-gradient operands end in a partial 5-row block."""
    _, ref, bf = case_and_oracle
    np.testing.assert_array_equal(ref[name], bf[name], err_msg=name)


@pytest.mark.parametrize("wrong,tensor", [("G:Wgu", "H"), ("Y:Wd", "Y"), ("Y:H", "Y"), ("dH:Wd", "dH"),
                                          ("dWd:dY", "dW_down"), ("dX:Wgu", "dX"), ("dWgu:X", "dW_gu")])
def test_mx_composition_wrong_axis_is_detected(case_and_oracle, wrong, tensor):
    """Negative control: one operand quantised along the wrong axis changes the tensor, so an
    oracle with that mistake fails the brute-force comparison above."""
    c, ref, _ = case_and_oracle
    alt = brute(c, wrong)
    assert not np.array_equal(alt[tensor], ref[tensor]), f"{wrong} left {tensor} unchanged"


def test_mx_composition_group_boundaries_in_layer_backward():
    """Two groups in one layer: the weight-gradient blocks restart at each group's first row
    (a block never straddles groups), so each group's dW equals its own brute force."""
    g = np.random.Generator(np.random.PCG64(9))
    T, d, f, E = 45, 64, 32, 2
    X = O.round_bf16(g.standard_normal((T, d)))
    Wgu = O.round_bf16(g.standard_normal((E, 2 * f, d)) * 0.02)
    Wd = O.round_bf16(g.standard_normal((E, d, f)) * 0.02)
    idx = np.where(np.arange(T)[:, None] < 40, 0, 1).astype(np.int32)   # groups of 40 and 5 rows
    w = np.ones((T, 1))
    fwd = O.layer_forward(X, None, None, 1, "softmax", lambda e: Wgu[e], lambda e: Wd[e], E,
                          rnd=O.round_bf16, topk=(idx, w), mx=True)
    dO = O.round_bf16(g.standard_normal((T, d)))
    bwd = O.layer_backward(fwd, dO, lambda e: Wgu[e], lambda e: Wd[e], E, rnd=O.round_bf16, mx=True)
    off = fwd["offsets"]
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        c = Case.__new__(Case)
        c.m, c.d, c.f = hi - lo, d, f
        c.X, c.Wgu, c.Wd = X[fwd["src_token"][lo:hi]], Wgu[e], Wd[e]
        c.dY = O.round_bf16(dO[fwd["src_token"][lo:hi]])      # weight one: dY row = d_out row
        ref = brute(c)
        np.testing.assert_array_equal(bwd["dW_gu"][e], ref["dW_gu"])
        np.testing.assert_array_equal(bwd["dW_down"][e], ref["dW_down"])
        np.testing.assert_array_equal(fwd["Y"][lo:hi], ref["Y"])


def test_mx_output_moves_past_6e2_when_one_intermediate_moves_one_bf16_ulp():
    """Why the whole MXFP8 step is gated on a high quantile rather than on its single worst
    element. The quantiser is discontinuous: moving one bf16 element of H by one ulp (within
    the bf16 gate of the stage that writes H) can flip its E4M3 code or its block's scale,
    and H = silu(G)*U is heavy-tailed, so the flipped element can be many times the rms of H.
    Here one such nudge moves an element of Y = rnd(Q(H) Q(W_down)^T) by more than 6e-2 of
    the rms of Y (the error metric e = |y - r| / max(|r|, rms(r))). Any implementation whose
    bf16 intermediates are not bit-identical to the oracle's can therefore exceed 6e-2 on a
    few elements of the step's outputs while every stage is correct."""
    g = np.random.Generator(np.random.PCG64(5))
    m, d, f = 256, 384, 256
    X = O.round_bf16(g.standard_normal((m, d)))
    Wgu = O.round_bf16(g.standard_normal((2 * f, d)) * 0.02)
    Wd = O.round_bf16(g.standard_normal((d, f)) * 0.02)
    H, Y = O.expert_forward(X, Wgu, Wd, O.round_bf16, mx=True)
    WdQ = O.mx_q_rows(Wd)
    HQ = O.mx_q_rows(H)
    rms = np.sqrt(np.mean(Y * Y))
    worst = 0.0
    for i in range(m):
        for n in np.argsort(-np.abs(H[i]))[:8]:           # the row's largest elements
            for sgn in (-1.0, 1.0):
                h = H[i, n]
                ulp = 2.0 ** (np.frexp(abs(h))[1] - 8)
                hp = O.round_bf16(h + sgn * ulp)            # the neighbouring bf16 value
                assert 0 < abs(hp - h) <= abs(h) * 2.0 ** -7
                row = H[i].copy()
                row[n] = hp
                q = O.mx_q_rows(row[None])[0]
                if np.array_equal(q, HQ[i]):
                    continue
                yp = O.round_bf16(q @ WdQ.T)
                worst = max(worst, float(np.max(np.abs(yp - Y[i]) / np.maximum(np.abs(Y[i]), rms))))
    assert worst > 6e-2, worst


# ---- MXFP4 forward ([OCP-MX] E2M1 elements, E8M0 scale floor(log2 amax) - 2)

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def q4_block(vals):
    """One MXFP4 block by brute force: scale 2^(floor(log2 amax) - 2) read off the block's
    largest magnitude with math.frexp, every element the nearest signed grid value by
    exhaustive search (ties to the grid value whose index is even, i.e. the even mantissa),
    magnitudes past 6 saturating."""
    vals = [float(v) for v in vals]
    amax = max(abs(v) for v in vals)
    if amax == 0.0:
        return np.zeros(len(vals))
    e = math.frexp(amax)[1] - 1 - 2
    X = 2.0 ** e
    out = []
    for v in vals:
        a = abs(v) / X
        dist = [abs(a - g) for g in E2M1_GRID]
        best = min(dist)
        idx = [i for i, dd in enumerate(dist) if dd == best]
        i = idx[0] if len(idx) == 1 else [j for j in idx if j % 2 == 0][0]
        out.append(math.copysign(E2M1_GRID[i] * X, v))
    return np.array(out)


def q4_vec(vec):
    vec = np.asarray(vec, np.float64)
    return np.concatenate([q4_block(vec[s:s + BLK]) for s in range(0, len(vec), BLK)])


def brute_mx4_forward(c: Case, wrong: str = ""):
    """H and Y of the MXFP4 expert forward, element by element: G and U contract over d (X
    rows and W_gu rows blocked along d), Y over f (H rows and W_down rows blocked along f).
    `wrong`: "G:Wgu" blocks W_gu along 2f, "Y:H" blocks H along the tokens, "Y:Wd" blocks
    W_down along d."""
    m, d, f = c.m, c.d, c.f
    Xq = [q4_vec(c.X[i]) for i in range(m)]
    if wrong == "G:Wgu":
        cols = [q4_vec(c.Wgu[:, j]) for j in range(d)]
        Wguq = [np.array([cols[j][r] for j in range(d)]) for r in range(2 * f)]
    else:
        Wguq = [q4_vec(c.Wgu[r]) for r in range(2 * f)]
    G = np.array([[dot(Xq[i], Wguq[n]) for n in range(f)] for i in range(m)])
    U = np.array([[dot(Xq[i], Wguq[f + n]) for n in range(f)] for i in range(m)])
    H = np.array([[rnd(silu(G[i, n]) * U[i, n]) for n in range(f)] for i in range(m)])
    if wrong == "Y:H":
        hc = [q4_vec(H[:, n]) for n in range(f)]
        Hq = [np.array([hc[n][i] for n in range(f)]) for i in range(m)]
    else:
        Hq = [q4_vec(H[i]) for i in range(m)]
    if wrong == "Y:Wd":
        wc = [q4_vec(c.Wd[:, n]) for n in range(f)]
        Wdq = [np.array([wc[n][e] for n in range(f)]) for e in range(d)]
    else:
        Wdq = [q4_vec(c.Wd[e]) for e in range(d)]
    Y = np.array([[rnd(dot(Hq[i], Wdq[e])) for e in range(d)] for i in range(m)])
    return dict(H=H, Y=Y)


@pytest.fixture(scope="module")
def mx4_case():
    c = Case(m=40, seed=11)
    H, Y = O.expert_forward(c.X, c.Wgu, c.Wd, O.round_bf16, mx4=True)
    return c, dict(H=H, Y=Y)


def test_mx4_forward_composition_matches_blockwise_brute_force(mx4_case):
    c, ref = mx4_case
    bf = brute_mx4_forward(c)
    np.testing.assert_array_equal(ref["H"], bf["H"])
    np.testing.assert_array_equal(ref["Y"], bf["Y"])


@pytest.mark.parametrize("wrong,tensor", [("G:Wgu", "H"), ("Y:H", "Y"), ("Y:Wd", "Y")])
def test_mx4_forward_wrong_axis_is_detected(mx4_case, wrong, tensor):
    c, ref = mx4_case
    alt = brute_mx4_forward(c, wrong)
    assert not np.array_equal(alt[tensor], ref[tensor]), f"{wrong} left {tensor} unchanged"


def test_mx4_layer_forward_uses_the_fp4_quantiser():
    """The layer forward's MXFP4 flag reaches every expert: its Y rows equal the per-expert
    MXFP4 forward on the gathered rows, and differ from the MXFP8 layer's."""
    g = np.random.Generator(np.random.PCG64(13))
    T, d, f, E = 24, 64, 32, 3
    X = O.round_bf16(g.standard_normal((T, d)))
    Wgu = O.round_bf16(g.standard_normal((E, 2 * f, d)) * 0.02)
    Wd = O.round_bf16(g.standard_normal((E, d, f)) * 0.02)
    idx = (np.arange(T) % E).astype(np.int32)[:, None]
    w = np.ones((T, 1))
    kw = dict(rnd=O.round_bf16, topk=(idx, w))
    f4 = O.layer_forward(X, None, None, 1, "softmax", lambda e: Wgu[e], lambda e: Wd[e], E, mx4=True, **kw)
    f8 = O.layer_forward(X, None, None, 1, "softmax", lambda e: Wgu[e], lambda e: Wd[e], E, mx=True, **kw)
    off = f4["offsets"]
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        c = Case.__new__(Case)
        c.m, c.d, c.f = hi - lo, d, f
        c.X, c.Wgu, c.Wd = X[f4["src_token"][lo:hi]], Wgu[e], Wd[e]
        np.testing.assert_array_equal(f4["Y"][lo:hi], brute_mx4_forward(c)["Y"])
    assert not np.array_equal(f4["Y"], f8["Y"])
