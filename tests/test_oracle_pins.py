"""Pins for the oracle: each check ties it to something other than itself (brute force,
closed forms, library routines, invariants, published format tables), chosen so that a
plausible mistake (a dropped term, a wrong sign or index, a transposed operand, a wrong
tie-break or rounding rule) fails at least one of them. CPU only."""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import moe_inputs as mi
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- roundings

def _all_bf16_values():
    bits = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16)
    v = bits.view(torch.bfloat16).float().double().numpy()
    ok = np.isfinite(v)
    return v[ok], np.arange(65536)[ok]


def test_round_bf16_matches_torch_on_fp32_inputs():
    g = np.random.Generator(np.random.PCG64(5))
    x = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-30, 30, 20000),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 3e38])]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(O.round_bf16(x.astype(np.float64)), want)


def test_round_bf16_brute_force_nearest_on_fp64_inputs():
    """Nearest of all finite bf16 values by exhaustive search; ties to the even code."""
    vals, codes = _all_bf16_values()
    order = np.argsort(vals, kind="stable")
    vals, codes = vals[order], codes[order]
    g = np.random.Generator(np.random.PCG64(6))
    x = g.standard_normal(3000) * 10.0 ** g.integers(-5, 5, 3000)
    # exact midpoints between neighbouring bf16 values (fp64 can hold them exactly)
    i = g.integers(40000 // 2, 65000 // 2, 200)
    mids = (vals[i] + vals[i + 1]) / 2
    for v in np.concatenate([x, mids]):
        dist = np.abs(vals - v)
        best = np.flatnonzero(dist == dist.min())
        cand = [c for c in best if vals[c] != 0 or True]
        if len(cand) > 1:
            # tie: the one whose bf16 code has an even mantissa LSB
            even = [c for c in cand if (codes[c] & 1) == 0]
            want = vals[even[0]]
        else:
            want = vals[cand[0]]
        got = O.round_bf16(np.array([v]))[0]
        assert got == want, (v, got, want)


# ----------------------------------------------------------------------------- routing

def _tiny_router(seed=0, T=24, d=16, E=6):
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((T, d)).astype(np.float32)
    w = (g.standard_normal((E, d)) * 0.3).astype(np.float32)
    b = (g.standard_normal(E) * 0.2).astype(np.float32)
    return x, w, b


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_route_matches_per_token_brute_force(score):
    x, w, b = _tiny_router(1)
    T, E, k = x.shape[0], w.shape[0], 3
    idx, wt, keys = O.route(x, w, b, k, score)
    for t in range(T):
        kap = []
        for e in range(E):
            L = math.fsum(float(x[t, i]) * float(w[e, i]) for i in range(x.shape[1]))
            kap.append(float(np.float32(np.float32(L) + np.float32(b[e]))))
        chosen = []
        for _ in range(k):                       # repeated argmax, lowest id on ties
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or kap[e] > kap[best]:
                    best = e
            chosen.append(best)
        assert list(idx[t]) == chosen
        if score == "softmax":
            full = [math.exp(v) for v in kap]                 # softmax over ALL experts ...
            p = [full[e] / sum(full) for e in range(E)]
            s = sum(p[e] for e in chosen)                     # ... renormalised over top-k
            want = [p[e] / s for e in chosen]
        else:
            sg = [1 / (1 + math.exp(-kap[e])) for e in chosen]
            want = [v / sum(sg) for v in sg]
        np.testing.assert_allclose(wt[t], want, rtol=1e-12, atol=0)


@pytest.mark.parametrize("name", ["small_softmax", "small_sigmoid", "tiny"])
def test_route_invariants(name):
    w = mi.WORKLOADS[name]
    x, wr, b = mi.x_np(w), mi.w_router_np(w), mi.expert_bias(w)
    idx, wt, keys = O.route(x, wr, b, w.k, w.score)
    assert idx.shape == (w.T, w.k)
    for t in range(w.T):
        assert len(set(idx[t].tolist())) == w.k
    assert np.bincount(idx.reshape(-1), minlength=w.E).sum() == w.T * w.k
    np.testing.assert_allclose(wt.sum(1), 1.0, atol=1e-12)
    assert np.all(np.diff(wt, axis=1) <= 0)
    kk = np.take_along_axis(keys, idx, 1)
    assert np.all(np.diff(kk, axis=1) <= 0)
    # every unselected key is <= the smallest selected one
    mask = np.ones_like(keys, dtype=bool)
    np.put_along_axis(mask, idx, False, 1)
    assert np.all(np.where(mask, keys, -np.inf).max(1) <= kk[:, -1])


def test_route_big_bias_takes_every_token():
    x, w, b = _tiny_router(2)
    b = np.zeros_like(b)
    b[4] = 100.0
    idx, _, _ = O.route(x, w, b, 2, "softmax")
    assert np.all(idx[:, 0] == 4)


def test_route_k_equals_E_is_full_softmax():
    x, w, b = _tiny_router(3)
    idx, wt, keys = O.route(x, w, b, w.shape[0], "softmax")
    p = scipy.special.softmax(keys.astype(np.float64), axis=1)
    np.testing.assert_allclose(wt, np.take_along_axis(p, idx, 1), rtol=1e-12)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_route_all_equal_keys_tie_break(score):
    x = np.zeros((5, 8), np.float32)
    w = np.ones((7, 8), np.float32)
    idx, wt, _ = O.route(x, w, None, 3, score)
    assert np.all(idx == np.arange(3))
    np.testing.assert_allclose(wt, 1 / 3, rtol=1e-15)


def test_route_integer_inputs_have_exact_keys():
    x = mi.integer_valued((50, 64), -2, 2, 0, 1)
    w = mi.integer_valued((9, 64), -1, 1, -4, 2)
    keys = O.router_keys(x, w, None)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    np.testing.assert_array_equal(keys.astype(np.float64), exact)


# ----------------------------------------------------------------------------- permutation

def _random_topk(T, E, k, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k", [(37, 5, 2), (64, 16, 4), (100, 8, 8), (1, 3, 1)])
def test_permutation_double_loop(T, E, k):
    idx = _random_topk(T, E, k, T + E)
    offsets, row_of, src = O.permutation(idx, E)
    want_src, want_row = [], np.full((T, k), -1)
    want_off = [0]
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    want_row[t, j] = len(want_src)
                    want_src.append(t)
        want_off.append(len(want_src))
    np.testing.assert_array_equal(offsets, want_off)
    np.testing.assert_array_equal(row_of, want_row)
    np.testing.assert_array_equal(src, want_src)


def test_permutation_invariants_and_shared_group():
    T, E, k = 200, 12, 3
    idx = _random_topk(T, E, k, 9)
    g = np.random.Generator(np.random.PCG64(19))
    others = np.array([e for e in range(E) if e != 7])
    for t in range(150):                                 # a hot expert
        idx[t] = np.concatenate([[7], g.permutation(others)[:k - 1]])
    for t in range(T):
        assert len(set(idx[t])) == k
    offsets, row_of, src = O.permutation(idx, E, shared_rows=T)
    assert len(offsets) == E + 2 and offsets[E] == T * k and offsets[E + 1] == T * k + T
    assert np.all(np.diff(offsets) >= 0)
    assert sorted(row_of.reshape(-1).tolist()) == list(range(T * k))
    for t in range(T):
        for j in range(k):
            assert src[row_of[t, j]] == t
            assert offsets[idx[t, j]] <= row_of[t, j] < offsets[idx[t, j] + 1]
    for e in range(E):
        seg = src[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
    np.testing.assert_array_equal(src[T * k:], np.arange(T))


# ----------------------------------------------------------------------------- combine / adjoints

@pytest.mark.parametrize("k", [2, 8])
def test_combine_of_permute_with_equal_weights_is_identity(k):
    T, E, d = 40, 16, 24
    x = mi.randn_np(0, 0, 0, T, d, 1.0, "bf16")
    idx = _random_topk(T, E, k, k)
    _, row_of, src = O.permutation(idx, E)
    xp = O.gather_rows(x, src)
    out = O.combine(xp, np.full((T, k), 1.0 / k), row_of, None, rnd=O.round_bf16)
    np.testing.assert_array_equal(out, x.astype(np.float64))


def test_adjoint_identities():
    g = np.random.Generator(np.random.PCG64(4))
    T, E, k, d = 30, 7, 3, 11
    idx = _random_topk(T, E, k, 4)
    _, row_of, src = O.permutation(idx, E)
    w = g.random((T, k))
    Y = g.standard_normal((T * k, d))
    dO = g.standard_normal((T, d))
    lhs = np.sum(O.combine(Y, w, row_of) * dO)
    dY, _ = O.combine_backward(dO, Y, w, row_of)
    assert abs(lhs - np.sum(Y * dY)) <= 1e-12 * abs(lhs)
    x = g.standard_normal((T, d))
    Z = g.standard_normal((T * k, d))
    lhs = np.sum(O.gather_rows(x, src) * Z)
    rhs = np.sum(x * O.permute_backward(Z, row_of))
    assert abs(lhs - rhs) <= 1e-12 * abs(lhs)


# ----------------------------------------------------------------------------- experts / GEMM

def test_silu_closed_form():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(O.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0
    h = 1e-6
    num = (O.silu(z + h) - O.silu(z - h)) / (2 * h)
    np.testing.assert_allclose(O.silu_grad(z), num, rtol=1e-6, atol=1e-9)


def test_grouped_gemm_single_group_is_dense_matmul():
    g = np.random.Generator(np.random.PCG64(8))
    A = g.standard_normal((33, 40))
    W = g.standard_normal((1, 24, 40))
    np.testing.assert_allclose(O.grouped_gemm(A, W, [0, 33]), np.matmul(A, W[0].T), rtol=1e-14)


def test_grouped_gemm_integer_exact_and_metamorphic():
    A = mi.integer_valued((70, 64), -2, 2, 0, 3)
    W = mi.integer_valued((4, 48, 64), -2, 2, -3, 4)
    off = [0, 0, 33, 34, 70]                         # empty group, 1-row group, ragged
    C = O.grouped_gemm(A, W, off)
    for g_, (lo, hi) in enumerate(zip(off[:-1], off[1:])):
        for r in range(lo, hi):
            for n in range(0, 48, 7):
                assert C[r, n] == sum(float(A[r, i]) * float(W[g_, n, i]) for i in range(64))
    np.testing.assert_array_equal(O.grouped_gemm(A, 2 * W, off), 2 * C)
    perm = np.random.Generator(np.random.PCG64(1)).permutation(70)
    inv = np.argsort(perm)
    np.testing.assert_array_equal(O.grouped_gemm(A[perm], W, off, a_row_index=inv), C)


def test_grouped_swiglu_matches_two_gemms():
    g = np.random.Generator(np.random.PCG64(9))
    A = g.standard_normal((20, 16))
    W = g.standard_normal((2, 10, 16))
    H = O.grouped_swiglu(A, W, [0, 7, 20])
    for lo, hi, e in [(0, 7, 0), (7, 20, 1)]:
        Gm = A[lo:hi] @ W[e, :5].T
        Um = A[lo:hi] @ W[e, 5:].T
        np.testing.assert_allclose(H[lo:hi], Gm * scipy.special.expit(Gm) * Um, rtol=1e-13)


# ----------------------------------------------------------------------------- whole layer

def _tiny_layer(seed, T=12, d=16, f=8, E=5, shared=True):
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((T, d))
    wr = g.standard_normal((E, d)) * 0.5
    b = g.standard_normal(E) * 0.1
    Wgu = g.standard_normal((E + 1, 2 * f, d)) * 0.3
    Wd = g.standard_normal((E + 1, d, f)) * 0.3
    return x, wr, b, Wgu, Wd


@pytest.mark.parametrize("score,k", [("softmax", 2), ("sigmoid", 3)])
def test_layer_matches_per_token_brute_force(score, k):
    x, wr, b, Wgu, Wd = _tiny_layer(10)
    E = wr.shape[0]
    fwd = O.layer_forward(x, wr, b, k, score, lambda e: Wgu[e], lambda e: Wd[e], E, shared=True)
    ref = O.layer_forward_per_token(x, wr, b, k, score, lambda e: Wgu[e], lambda e: Wd[e], E, shared=True)
    np.testing.assert_allclose(fwd["out"], ref, rtol=1e-12, atol=1e-12)


def test_layer_identical_experts_gives_dense_mlp():
    x, wr, b, Wgu, Wd = _tiny_layer(11)
    E = wr.shape[0]
    fwd = O.layer_forward(x, wr, b, 3, "sigmoid", lambda e: Wgu[0], lambda e: Wd[0], E, shared=False)
    G, U = x @ Wgu[0][:8].T, x @ Wgu[0][8:].T
    dense = (G * scipy.special.expit(G) * U) @ Wd[0].T
    np.testing.assert_allclose(fwd["out"], dense, rtol=1e-12, atol=1e-13)


def test_layer_single_expert_is_dense_swiglu():
    x, wr, b, Wgu, Wd = _tiny_layer(12, E=1)
    fwd = O.layer_forward(x, wr, None, 1, "softmax", lambda e: Wgu[e], lambda e: Wd[e], 1)
    G, U = x @ Wgu[0][:8].T, x @ Wgu[0][8:].T
    np.testing.assert_allclose(fwd["out"], (G * scipy.special.expit(G) * U) @ Wd[0].T, rtol=1e-12, atol=1e-13)


def test_layer_token_permutation_equivariance():
    x, wr, b, Wgu, Wd = _tiny_layer(13)
    E = wr.shape[0]
    run = lambda xx: O.layer_forward(xx, wr, b, 2, "softmax", lambda e: Wgu[e], lambda e: Wd[e], E,
                                     shared=True, rnd=O.round_bf16)["out"]
    perm = np.random.Generator(np.random.PCG64(2)).permutation(x.shape[0])
    np.testing.assert_array_equal(run(x)[perm], run(x[perm]))


# ----------------------------------------------------------------------------- MXFP8

def _golden_mx():
    rows = []
    for line in open(os.path.join(GOLDEN, "mx_e4m3_cases.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        amax, sb, el, scaled, code = line.split()
        rows.append((eval(amax), int(sb), eval(el), float(scaled), int(code, 16)))
    return rows


def test_mx_golden_cases():
    rows = _golden_mx()
    assert len(rows) >= 10
    for amax, sb, el, scaled, code in rows:
        block = np.zeros(32)
        block[0] = amax
        block[5] = el
        codes, sbs, dq = O.mx_quantize_blocks(block[None])
        assert int(sbs[0]) == sb, (amax, sbs)
        X = 2.0 ** (sb - 127)
        assert el / X == pytest.approx(scaled, rel=1e-15)
        assert int(codes[0, 5]) == code, (amax, el, hex(int(codes[0, 5])))
        assert O.e4m3_decode(codes[0, 5]) * X == dq[0, 5]


def test_mx_zero_block():
    codes, sb, dq = O.mx_quantize_blocks(np.zeros((3, 32)))
    assert np.all(sb == 0) and np.all(codes == 0) and np.all(dq == 0)


def test_e4m3_matches_torch_in_range():
    g = np.random.Generator(np.random.PCG64(7))
    v = np.concatenate([g.uniform(-448, 448, 20000), g.standard_normal(20000) * 2.0 ** -7,
                        np.array([448.0, -448.0, 2 ** -9, 2 ** -10, 3 * 2 ** -11, 0.0])])
    v32 = v.astype(np.float32).astype(np.float64)
    want = torch.from_numpy(v32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_encode(O.e4m3_round(v32)), want)


def test_e4m3_every_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = O.e4m3_decode(codes)
    np.testing.assert_array_equal(O.e4m3_encode(O.e4m3_round(vals)), codes)
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(vals, tv)


def test_mx_values_on_grid_are_fixed_points():
    ints = mi.integer_valued((6, 64), -3, 3, -5, 11).astype(np.float64)
    ints[:, ::32] = 3 * 2.0 ** -5                     # every block holds its max
    np.testing.assert_array_equal(O.mx_q_rows(ints), ints)


def test_mx_colwise_grouped_equals_rowwise_of_padded_transpose():
    g = np.random.Generator(np.random.PCG64(12))
    a = g.standard_normal((101, 40)) * np.exp(g.standard_normal((101, 1)))
    off = [0, 33, 33, 34, 101]                          # partial blocks, empty, 1-row group
    codes, scales, dq = O.mx_quantize_colwise_grouped(a, off)
    for gi, (lo, hi) in enumerate(zip(off[:-1], off[1:])):
        m = hi - lo
        nb = -(-m // 32)
        pad = np.zeros((40, nb * 32))
        pad[:, :m] = a[lo:hi].T
        c2, s2, d2 = O.mx_quantize_rowwise(pad)
        np.testing.assert_array_equal(codes[lo:hi], c2[:, :m].T)
        np.testing.assert_array_equal(scales[gi], s2.T)
        np.testing.assert_array_equal(dq[lo:hi], d2[:, :m].T)


# ----------------------------------------------------------------------------- backward

def test_backward_matches_finite_differences():
    x, wr, b, Wgu, Wd = _tiny_layer(14, T=6, d=5, f=3, E=3)
    E, k = 3, 2
    idx, w, _ = O.route(x, wr, b, k, "softmax")
    g = np.random.Generator(np.random.PCG64(3))
    dO = g.standard_normal(x.shape)

    def loss(xx, Wgu_, Wd_):
        f = O.layer_forward(xx, wr, b, k, "softmax", lambda e: Wgu_[e], lambda e: Wd_[e], E,
                            shared=True, topk=(idx, w))
        return np.sum(f["out"] * dO)

    fwd = O.layer_forward(x, wr, b, k, "softmax", lambda e: Wgu[e], lambda e: Wd[e], E, shared=True,
                          topk=(idx, w))
    bwd = O.layer_backward(fwd, dO, lambda e: Wgu[e], lambda e: Wd[e], E, shared=True)
    h = 1e-6
    for (t, i) in [(0, 0), (3, 4), (5, 2)]:
        xp, xm = x.copy(), x.copy()
        xp[t, i] += h
        xm[t, i] -= h
        num = (loss(xp, Wgu, Wd) - loss(xm, Wgu, Wd)) / (2 * h)
        assert bwd["dx"][t, i] == pytest.approx(num, rel=1e-6, abs=1e-9)
    for (e, n, i) in [(0, 1, 2), (1, 5, 0), (3, 2, 4)]:
        Wp, Wm = Wgu.copy(), Wgu.copy()
        Wp[e, n, i] += h
        Wm[e, n, i] -= h
        num = (loss(x, Wp, Wd) - loss(x, Wm, Wd)) / (2 * h)
        assert bwd["dW_gu"][e][n, i] == pytest.approx(num, rel=1e-6, abs=1e-9)
        Wp, Wm = Wd.copy(), Wd.copy()
        Wp[e, i, n % 3] += h
        Wm[e, i, n % 3] -= h
        num = (loss(x, Wgu, Wp) - loss(x, Wgu, Wm)) / (2 * h)
        assert bwd["dW_down"][e][i, n % 3] == pytest.approx(num, rel=1e-6, abs=1e-9)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_layer_backward_with_router_matches_finite_differences(score):
    """The whole layer, routing included: the loss's gradients with respect to the input, the
    router weights and the expert bias, by central differences with the routing recomputed
    at every point (the keys' top-k margin is far above the step, so the selection holds).
    The keys are stored in fp32, so x, the router weights, the bias and the step are dyadic
    with few bits: every perturbed key is then exact and the differences carry no rounding."""
    x, wr, b, Wgu, Wd = _tiny_layer(16, T=6, d=5, f=3, E=4)
    x, wr, b = np.round(x * 8) / 8, np.round(wr * 16) / 16, np.round(b * 64) / 64
    E, k = 4, 2
    dO = np.random.Generator(np.random.PCG64(5)).standard_normal(x.shape)
    gu, dn = (lambda e: Wgu[e]), (lambda e: Wd[e])

    def loss(xx, wr_, b_):
        return np.sum(O.layer_forward(xx, wr_, b_, k, score, gu, dn, E, shared=True)["out"] * dO)

    fwd = O.layer_forward(x, wr, b, k, score, gu, dn, E, shared=True)
    h = 2.0 ** -12
    srt = -np.sort(-fwd["keys"].astype(np.float64), axis=1)
    assert np.min(srt[:, k - 1] - srt[:, k]) > 2 * h * max(np.abs(x).max(), np.abs(wr).max(), 1.0)
    bwd = O.layer_backward(fwd, dO, gu, dn, E, shared=True, router=(x, wr, score))

    def num(a, pos, f):
        ap, am = a.copy(), a.copy()
        ap[pos] += h
        am[pos] -= h
        return (f(ap) - f(am)) / (2 * h)

    for pos in [(0, 0), (3, 4), (5, 2)]:
        assert bwd["dx"][pos] == pytest.approx(num(x, pos, lambda a: loss(a, wr, b)), rel=1e-6, abs=1e-9)
    for pos in [(0, 1), (2, 3), (3, 0)]:
        assert bwd["dW_router"][pos] == pytest.approx(num(wr, pos, lambda a: loss(x, a, b)), rel=1e-6, abs=1e-9)
    for e in range(E):
        assert bwd["d_bias"][e] == pytest.approx(num(b, (e,), lambda a: loss(x, wr, a)), rel=1e-6, abs=1e-9)


def test_backward_empty_group_has_zero_weight_grad():
    x, wr, b, Wgu, Wd = _tiny_layer(15, d=64, f=32, E=4)
    idx = np.array([[0, 1]] * x.shape[0], np.int32)   # experts 2 and 3 empty
    w = np.full(idx.shape, 0.5)
    fwd = O.layer_forward(x, wr, b, 2, "softmax", lambda e: Wgu[e], lambda e: Wd[e], 4, topk=(idx, w))
    bwd = O.layer_backward(fwd, np.ones_like(x), lambda e: Wgu[e], lambda e: Wd[e], 4,
                           rnd=O.round_bf16, mx=True)
    for e in (2, 3):
        assert np.all(bwd["dW_gu"][e] == 0) and np.all(bwd["dW_down"][e] == 0)
    assert np.any(bwd["dW_gu"][0] != 0)


def test_mx_backward_on_grid_inputs_matches_plain_where_operands_are_on_grid():
    """With X, the weights and dY on the MX grid the quantiser is the identity on them, so
    every GEMM that reads only those operands must give the plain result exactly."""
    def grid(shape, log2s, seed):
        a = mi.integer_valued(shape, -3, 3, log2s, seed).astype(np.float64)
        a[:, ::32] = 3 * 2.0 ** log2s                  # each row block holds its max ...
        a[::32, :] = 3 * 2.0 ** log2s                  # ... and so does each column block
        return a
    X, Wgu, Wd, dY = grid((64, 64), -2, 21), grid((64, 64), -3, 22), grid((64, 32), -3, 23), grid((64, 64), -1, 24)
    for arr in (X, Wgu, Wd, dY):
        np.testing.assert_array_equal(O.mx_q_rows(arr), arr)
        np.testing.assert_array_equal(O.mx_q_rows(arr.T).T, arr)
    a = O.expert_backward(X, Wgu, Wd, dY, mx=True)
    b = O.expert_backward(X, Wgu, Wd, dY, mx=False)
    np.testing.assert_array_equal(a["G"], b["G"])
    np.testing.assert_array_equal(a["U"], b["U"])
    np.testing.assert_array_equal(a["dH"], b["dH"])


# ----------------------------------------------------------------------------- router backward

def _router_loss(x, wr, b, g, idx, score):
    """sum_tj g[t,j] w[t,j] with the pure fp64 keys x W_r^T + b and a fixed selection."""
    keys = x @ wr.T + b
    return float((g * O.topk_weights(keys, idx, score)).sum())


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_router_backward_matches_finite_differences(score):
    gen = np.random.Generator(np.random.PCG64(31))
    T, d, E, k = 5, 6, 7, 3
    x = gen.standard_normal((T, d))
    wr = gen.standard_normal((E, d)) * 0.5
    b = gen.standard_normal(E) * 0.3
    g = gen.standard_normal((T, k))
    keys = x @ wr.T + b
    idx = O.select_topk(keys, k)
    srt = -np.sort(-keys, axis=1)
    assert (srt[:, k - 1] - srt[:, k]).min() > 1e-3          # the selection cannot move under eps
    dkeys = O.topk_weights_backward(keys, idx, g, score)
    dW, dx, db = O.router_backward(x, wr, dkeys)
    eps = 1e-6
    for arr, grad in ((x, dx), (wr, dW), (b, db)):
        num = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            a0 = arr[i]
            arr[i] = a0 + eps
            lp = _router_loss(x, wr, b, g, idx, score)
            arr[i] = a0 - eps
            lm = _router_loss(x, wr, b, g, idx, score)
            arr[i] = a0
            num[i] = (lp - lm) / (2 * eps)
        assert np.abs(num - grad).max() <= 1e-7 * max(1.0, np.abs(num).max())
    # unselected experts get no gradient
    mask = np.zeros_like(keys, dtype=bool)
    np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
    assert np.all(dkeys[~mask] == 0.0)


def test_router_backward_softmax_k_equals_E_is_softmax_jacobian():
    # with every expert selected the weights are a plain softmax: d kappa = (diag(w) - w w^T) g
    gen = np.random.Generator(np.random.PCG64(32))
    T, E = 4, 6
    keys = gen.standard_normal((T, E))
    g = gen.standard_normal((T, E))
    idx = O.select_topk(keys, E)
    dk = O.topk_weights_backward(keys, idx, g, "softmax")
    for t in range(T):
        w = scipy.special.softmax(keys[t])
        J = np.diag(w) - np.outer(w, w)
        g_e = np.zeros(E)
        g_e[idx[t]] = g[t]                                  # weights are stored in selection order
        np.testing.assert_allclose(dk[t], J @ g_e, rtol=0, atol=1e-14)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_router_backward_invariants(score):
    gen = np.random.Generator(np.random.PCG64(33))
    T, E, k = 50, 16, 4
    keys = gen.standard_normal((T, E))
    idx = O.select_topk(keys, k)
    # a gradient equal on every selected weight changes nothing: the weights sum to one
    c = gen.standard_normal((T, 1)) * np.ones((1, k))
    assert np.abs(O.topk_weights_backward(keys, idx, c, score)).max() < 1e-15
    if score == "softmax":
        # a common shift of the selected keys leaves a softmax unchanged
        g = gen.standard_normal((T, k))
        assert np.abs(O.topk_weights_backward(keys, idx, g, score).sum(axis=1)).max() < 1e-14


# ----------------------------------------------------------------------------- MXFP4

def _golden_mx4():
    rows = []
    for line in open(os.path.join(GOLDEN, "mx_e2m1_cases.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        amax, sb, el, scaled, code = line.split()
        rows.append((eval(amax), int(sb), eval(el), float(scaled), int(code, 16)))
    return rows


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def test_mx4_golden_cases():
    rows = _golden_mx4()
    assert len(rows) >= 20
    for amax, sb, el, scaled, code in rows:
        block = np.zeros(32)
        block[0] = amax
        block[7] = el
        codes, sbs, dq = O.mx4_quantize_blocks(block[None])
        assert int(sbs[0]) == sb, (amax, sbs)
        X = 2.0 ** (sb - 127)
        assert el / X == pytest.approx(scaled, rel=1e-15)
        assert int(codes[0, 7]) == code, (amax, el, hex(int(codes[0, 7])))
        assert O.e2m1_decode(codes[0, 7]) * X == dq[0, 7]


def test_e2m1_every_code_round_trips_and_decodes_to_the_table():
    codes = np.arange(16, dtype=np.uint8)
    vals = O.e2m1_decode(codes)
    np.testing.assert_array_equal(np.abs(vals[:8]), E2M1_GRID)
    np.testing.assert_array_equal(vals[8:], -E2M1_GRID)
    np.testing.assert_array_equal(O.e2m1_encode(O.e2m1_round(vals)), codes)


def test_e2m1_round_is_nearest_with_ties_to_even_mantissa():
    """Brute force over the 8 magnitudes: the nearest one wins; at an exact midpoint the one
    with mantissa bit 0 (codes 0, 2, 4, 6); above 6 saturates."""
    g = np.random.Generator(np.random.PCG64(41))
    mids = (E2M1_GRID[:-1] + E2M1_GRID[1:]) / 2
    v = np.concatenate([g.uniform(-8, 8, 20000), mids, -mids, [6.0, 6.5, 100.0, 0.0]])
    got = O.e2m1_round(v)
    a = np.abs(v)
    dist = np.abs(a[:, None] - E2M1_GRID[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = np.where(dist == best, np.arange(8)[None, :], 99)
    even = np.where(cand % 2 == 0, cand, 99).min(axis=1)
    pick = np.where(even < 99, even, cand.min(axis=1))
    np.testing.assert_array_equal(np.abs(got), E2M1_GRID[pick])
    np.testing.assert_array_equal(np.signbit(got[a > 0.25]), np.signbit(v[a > 0.25]))


def test_mx4_values_on_grid_are_fixed_points():
    g = np.random.Generator(np.random.PCG64(42))
    vals = E2M1_GRID[g.integers(0, 8, (5, 64))] * np.where(g.random((5, 64)) < 0.5, -1, 1)
    vals[:, ::32] = 6.0                                  # every block holds its maximum
    a = vals * 2.0 ** -7
    np.testing.assert_array_equal(O.mx4_q_rows(a), a)
