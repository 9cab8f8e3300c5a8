"""CPU replay of the column-wise / dual quantiser's XCD-aware tile order (quant.hip,
quant_tile_of_block): for the grids the layer launches and a sweep of others, the launch
order -> (column tile, chunk) map is a bijection onto the grid, each XCD's workgroups take one
contiguous run of tiles, and the 8 column tiles of a row-wise scale sector's band run as
consecutive workgroups of one XCD. Mirrors the kernel's formula; a change there must be
mirrored here."""
import numpy as np
import pytest

import moe_inputs as mi

XCDS = 8
COL_TILE = 128          # bf16 columns per workgroup


def tile_of_block(X, Y):
    """(cx, cy) of every workgroup in launch order L = y X + x, as the kernel computes them."""
    L = np.arange(X * Y, dtype=np.int64)
    if X % 8:
        return L % X, L // X
    lam = (L % 8) * (X // 8 * Y) + L // 8
    band, rem = lam // (8 * Y), lam % (8 * Y)
    return band * 8 + rem % 8, rem // 8


def _grids():
    out = []
    for name in ("dsv3", "dsv3_mxfp8", "mixtral", "qwen3"):
        w = mi.WORKLOADS[name]
        for cols in (w.d, 2 * w.f, w.f):        # the weight stacks' K, and the activations' widths
            out.append((cols // COL_TILE, 8 + w.E))
    out += [(8, 1), (16, 3), (56, 7), (56, 8257), (64, 100), (24, 5)]
    return sorted(set(out))


@pytest.mark.parametrize("X,Y", _grids())
def test_quant_tile_order_is_a_bijection_with_xcd_runs(X, Y):
    cx, cy = tile_of_block(X, Y)
    assert cx.min() >= 0 and cx.max() < X and cy.min() >= 0 and cy.max() < Y
    assert len(set(zip(cx.tolist(), cy.tolist()))) == X * Y
    if X % 8:
        return
    L = np.arange(X * Y)
    per = X * Y // XCDS
    # position of each tile in the order band (8 column tiles), chunk, column tile in the band
    lam = (cx // 8) * (8 * Y) + cy * 8 + cx % 8
    for x in range(XCDS):
        # the workgroups the hardware deals to XCD x (every 8th in launch order) take one
        # contiguous run of that order, in launch order
        k = L[L % XCDS == x]
        assert np.array_equal(lam[k], np.arange(x * per, (x + 1) * per))
    # so each run of 8 positions (one chunk's 8 column tiles of a band, the writers of one
    # 32-byte row-wise scale sector per row) lies on a single XCD as consecutive workgroups
    # whenever the run does not straddle two XCDs' ranges
    owner = np.empty(X * Y, np.int64)
    owner[lam] = L % XCDS
    runs = owner.reshape(-1, 8)
    starts = np.arange(0, X * Y, 8)
    inside = starts // per == (starts + 7) // per
    assert np.all(runs[inside] == runs[inside][:, :1])
