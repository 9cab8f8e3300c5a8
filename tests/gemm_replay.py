"""Host-side replay of the grouped GEMM's integer index math (no floating point).

A line-by-line model, in numpy, of what moe_grouped_gemm's kernels compute from the group
offsets: the schedule kernel's tile prefix and group order, the persistent workgroups' walk
over the tile list (XCD-aware slots, binary search of the prefix, row-tile and column-tile
decomposition), and for every tile the byte ranges its load waves' DMA instructions read (A
rows through the gather index, B rows of the group, MXFP8 scale dwords, over every K slice),
the LDS bytes they fill, and the output elements the epilogue writes. bf16 launches that
split (gemm_split_kernel) take each group's full 256-row chunks as 256 x 256 tiles first (8
waves that each load 64 rows of a stage), then the usual row tiles with all 8 waves issuing
loads. It asserts that every
access stays inside its buffer and that every output element of every group is written by
exactly one tile, so a launch shape can be cleared on the CPU before it runs on a GPU.

Constants and formulas follow the kernel source (csrc/gemm.hip); a change there must be
mirrored here.
"""
from __future__ import annotations

import dataclasses

import numpy as np

WAVE = 64
L_WAVES = 4            # load-issuing waves
BN = 256               # B rows per tile
ROW_BYTES = 128        # one LDS row per stage
ROWS_PER_INSTR = 1024 // ROW_BYTES
MAX_GROUPS = 2047


def cdiv(a, b):
    return -(-a // b)


def stage_bytes(bm, fp4=False):
    sdw = 2 if fp4 else 1          # scale dwords per row and stage
    scale_rows_a = cdiv(bm, 64) * 64
    data = (bm + BN) * ROW_BYTES
    return dict(data=data, scale_a=data, scale_b=data + scale_rows_a * 4 * sdw, sdw=sdw, scale_rows_a=scale_rows_a,
                bytes=data + (scale_rows_a + BN) * 4 * sdw, count=2 if bm == 256 else 3)


PIPE_BYTES = max(3 * stage_bytes(128)["bytes"], 2 * stage_bytes(256)["bytes"])
LDS_BYTES = PIPE_BYTES + (MAX_GROUPS + 1) * 4
# block-scaled row tiles (MXFP8, MXFP4): operand stages of codes only, then two scale-batch
# slots of 16 bytes per A and B row (the scales of 4 MXFP8 or 2 MXFP4 stages), then the prefix
SC_BATCH_BYTES = 16
SC_PIECE = 16 * SC_BATCH_BYTES           # LDS bytes per 16-row piece
SC_SLOT = (cdiv(128, 64) * 64 + BN) // 16 * SC_PIECE
MX_DATA = 3 * stage_bytes(128)["data"]
MX_PIPE = MX_DATA + 2 * SC_SLOT
MAX_GROUPS_MX = (160 * 1024 - MX_PIPE) // 4 - 1
assert MAX_GROUPS_MX == 1023 and MX_PIPE + (MAX_GROUPS_MX + 1) * 4 <= 160 * 1024
assert LDS_BYTES <= 160 * 1024 and PIPE_BYTES + 8 * 1024 <= MX_PIPE + (MAX_GROUPS_MX + 1) * 4

# 256 x 256 tiles: two 64 KiB stages (256 A rows, then 256 B rows) and the bf16 output tile
# staged over them, all below the tile prefix
STAGE256 = 2 * 256 * ROW_BYTES
assert 2 * STAGE256 <= PIPE_BYTES and 256 * (BN * 2 + 16) <= PIPE_BYTES


# the host's split thresholds: smallest group whose 256-row chunks take 256 x 256 tiles, for K
# below SPLIT_LONGK and from it on
SPLIT_MIN_ROWS = 256
SPLIT_LONGK = 4096
SPLIT_MIN_ROWS_LONGK = 1024


def chunk256_rows(m, split_min):
    """Rows of a group that 256 x 256 tiles cover (its full 256-row chunks) when the launch
    splits (split_min: the smallest group that gets them; 0: no split)."""
    return (m & ~255) if (split_min and m >= split_min) else 0


def bm_of_rows(m):
    return 16 if m <= 16 else 32 if m <= 32 else 64 if m <= 64 else 128


def row_tiles(m, allow256=False):
    """(n256, n128, last) as the kernel's row_tiles."""
    if m <= 128:
        return (0, 0, bm_of_rows(m) if m > 0 else 0)
    rest, n256 = m, 0
    if allow256 and m >= 256:
        n256 = m // 256
        rest -= 256 * n256
    n128 = rest // 128
    rest -= 128 * n128
    return (n256, n128, bm_of_rows(rest) if rest > 0 else 0)


def rt_count(rt):
    return rt[0] + rt[1] + (1 if rt[2] > 0 else 0)


def row_tile(rt, mt):
    n256, n128, last = rt
    if mt < n256:
        return 256 * mt, 256
    if mt < n256 + n128:
        return 256 * n256 + 128 * (mt - n256), 128
    return 256 * n256 + 128 * n128, last


def tile_coords(L, MT, NT, sup=4):
    full = NT // sup
    if L < full * MT * sup:
        s, rem = divmod(L, MT * sup)
        return rem // sup, s * sup + rem % sup
    rem = L - full * MT * sup
    w = NT - full * sup
    return rem // w, full * sup + rem % w


def group_rows(offsets, g, M):
    b = min(max(int(offsets[g]), 0), M)
    e = min(max(int(offsets[g + 1]), b), M)
    return b, e


def schedule(offsets, G, M, NT, allow256=False, split=0):
    """tile_start [G+1] and order [G] as gemm_schedule_kernel writes them (split: a group's
    tiles are its 256-row chunks' tiles, then the row tiles of the rows past them)."""
    tiles = np.zeros(G, np.int64)
    small = np.zeros(G, bool)
    rows = np.zeros(G, np.int64)
    for g in range(G):
        b, e = group_rows(offsets, g, M)
        rows[g] = e - b
        c256 = chunk256_rows(e - b, split)
        tiles[g] = (c256 // 256 + rt_count(row_tiles(e - b - c256, allow256))) * NT
        small[g] = (e - b) <= 128
    tot_small = int(tiles[small].sum())
    tot_large = int(tiles[~small].sum())
    pre_small = np.cumsum(np.where(small, tiles, 0)) - np.where(small, tiles, 0)
    pre_large = np.cumsum(np.where(~small, tiles, 0)) - np.where(~small, tiles, 0)
    keys = []
    for g in range(G):
        if tiles[g] > 0:
            p = int(pre_small[g] if small[g] else pre_large[g])
            total = tot_small if small[g] else tot_large
            frac = ((2 * p + int(tiles[g])) << 23) // total
            first = (tot_small >= tot_large) if small[g] else (tot_large > tot_small)
            late = 0 if (allow256 and rows[g] >= 256) else 1
            k = (late << 60) | (frac << 32) | ((0 if first else 1) << 16) | g
        else:
            k = (0xFFFFFFF << 32) | (2 << 60) | g
        assert k < (1 << 64)
        keys.append(k)
    assert len(set(keys)) == G, "schedule keys must be distinct"
    order = np.array(sorted(range(G), key=lambda g: keys[g]), np.int64)
    ts = np.zeros(G + 1, np.int64)
    ts[1:] = np.cumsum(tiles[order])
    return ts, order


@dataclasses.dataclass
class Launch:
    """One ragged-row grouped GEMM launch as the host entry point sets it up."""
    offsets: np.ndarray     # [G+1]
    M: int                  # rows of C
    N: int                  # output columns
    K: int
    A_rows: int
    lda: int
    a_rows: np.ndarray | None
    b_groups: int           # groups the B buffer holds (B tensor's first dimension)
    ldb: int
    b_stride: int           # elements between groups' B
    b_bytes: int            # bytes of the B allocation reachable from its base
    ldc: int
    c_esize: int
    swiglu: bool
    mx: bool = False
    fp4: bool = False       # E2M1 operands (implies mx): leading dimensions and strides in elements, two per byte
    uniform_rows: int = 0   # the router's K-split mode: group g owns C rows [g R, (g+1) R), no schedule
    a_group_stride: int = 0
    lda_scale: int = 0
    ldb_scale: int = 0
    b_scale_stride: int = 0
    b_scale_bytes: int = 0
    aux_ld: int = 0
    num_cus: int = 256
    split256: int | None = None    # None: the host's rule (bf16, bf16 C, ragged rows, no row index,
                                   # no G|U save, M >= 256)


def splits(la) -> int:
    """The launch's split256 parameter: 0, or the smallest group with 256 x 256 tiles."""
    if la.split256 is not None:
        return la.split256
    if (not la.mx) and la.c_esize == 2 and la.uniform_rows == 0 and la.aux_ld == 0 and la.a_rows is None \
            and la.M >= 256:
        return max(SPLIT_MIN_ROWS_LONGK if la.K >= SPLIT_LONGK else SPLIT_MIN_ROWS, 256)
    return 0


def check_launch(la: Launch):
    """Replay the whole launch; raise AssertionError at the first access outside a buffer or
    at any output element not written exactly once. Returns a summary dict."""
    G = len(la.offsets) - 1
    if la.fp4:
        assert la.mx and la.lda % 2 == 0 and la.ldb % 2 == 0 and la.b_stride % 2 == 0
    if la.mx:
        assert G <= MAX_GROUPS_MX
    eb = 1 if la.mx else 2
    byt = (lambda e: e // 2) if la.fp4 else (lambda e: e * eb)
    assert 1 <= G <= MAX_GROUPS
    bn_out = BN // 2 if la.swiglu else BN
    NT = cdiv(la.N, bn_out)
    kps = 2 * ROW_BYTES if la.fp4 else ROW_BYTES // eb      # K elements per stage
    assert la.K % kps == 0
    nk = la.K // kps
    a_bytes = la.A_rows * byt(la.lda)
    # the host's 4 GiB rule for 32-bit lane offsets
    b_span = (2 if la.swiglu else 1) * la.N * byt(la.ldb)
    assert a_bytes + byt(la.K) < 1 << 32 and b_span + byt(la.K) < 1 << 32
    uniform = la.uniform_rows > 0
    if uniform:
        rt_u = row_tiles(la.uniform_rows)
        per_group_u = rt_count(rt_u) * NT
        total = G * per_group_u
        tiles = total
        grid = min(la.num_cus, tiles)
    else:
        split = splits(la)
        ts, order = schedule(la.offsets, G, la.M, NT, split=split)
        total = int(ts[G])
        bound = (la.M // 16 + G) * NT
        grid = min(la.num_cus, max(bound, 1))
    nxcd = 8 if grid % 8 == 0 else 1
    per_xcd = grid // nxcd
    written = np.zeros((la.M, NT), np.int32)     # tiles covering each (row, column tile)
    seen_tiles = total256 = 0
    lwaves = 8 if (not uniform and split) else L_WAVES   # the split kernel has no producer waves
    for bid in range(grid):
        slot = (bid % nxcd) * per_xcd + bid // nxcd
        for tile in range(slot, total, grid):
            seen_tiles += 1
            if uniform:
                g, L = divmod(tile, per_group_u)
                rb = min(g * la.uniform_rows, la.M)
                re = min(rb + la.uniform_rows, la.M)
                rt = rt_u
            else:
                lo, hi = 0, G - 1
                while lo < hi:
                    mid = (lo + hi + 1) >> 1
                    if ts[mid] <= tile:
                        lo = mid
                    else:
                        hi = mid - 1
                g = min(max(int(order[lo]), 0), G - 1)
                L = tile - int(ts[lo])
                rb, re = group_rows(la.offsets, g, la.M)
                c256 = chunk256_rows(re - rb, split)
                t256 = c256 // 256 * NT
                if L < t256:
                    mt, nt = tile_coords(L, c256 // 256, NT)
                    assert 0 <= mt < c256 // 256 and 0 <= nt < NT, (tile, g, mt, nt)
                    _check_tile256(la, g, rb, re, rb + 256 * mt, nt, nk, written)
                    total256 += 1
                    continue
                L -= t256
                rt = row_tiles(re - rb - c256)
            mt, nt = tile_coords(L, rt_count(rt), NT)
            assert 0 <= mt < rt_count(rt) and 0 <= nt < NT, (tile, g, mt, nt)
            r_off, bm = row_tile(rt, mt)
            if not uniform:
                r_off += c256
            assert bm in (16, 32, 64, 128)
            _check_tile(la, g, rb, re, r_off, bm, nt, nk, byt, written, lwaves)
    assert seen_tiles == total
    # every row of every group: each column tile written exactly once; other rows untouched
    live = np.zeros(la.M, bool)
    for g in range(G):
        if uniform:
            b = min(g * la.uniform_rows, la.M)
            e = min(b + la.uniform_rows, la.M)
        else:
            b, e = group_rows(la.offsets, g, la.M)
        live[b:e] = True
    assert np.all(written[live] == 1), "an output element of a group was not written exactly once"
    assert np.all(written[~live] == 0), "a row outside every group was written"
    return dict(grid=grid, tiles=total, nk=nk, NT=NT, tiles256=total256)


def _check_tile256(la, g, row_begin, row_end, r0, nt, nk, written):
    """One gemm256_kernel tile: waves 0-3 load A rows, 4-7 B rows, 64 per wave and stage in 8
    instructions of 8 rows x 128 bytes; SwiGLU B rows pair 64 gate and 64 up rows per
    128-row half; bf16 output staged in LDS."""
    lane = np.arange(WAVE)
    WTN = 128
    bn_out = BN // 2 if la.swiglu else BN
    n0 = nt * bn_out
    k_extent = (nk - 1) * ROW_BYTES + 16
    a_bytes = la.A_rows * la.lda * 2
    b_base = g * la.b_stride * 2
    for wave in range(8):
        loads_a = wave < 4
        lrow0 = (wave % 4) * 64
        for i in range(8):
            row = lrow0 + 8 * i + lane // 8
            chunk = (lane % 8) ^ ((row >> 1) & 7)
            if loads_a:
                r = np.minimum(r0 + row, row_end - 1)
                ar = la.a_rows[r].astype(np.int64) if la.a_rows is not None else r.astype(np.int64)
                ar = np.clip(ar, 0, la.A_rows - 1)
                voff = ar * la.lda * 2 + chunk * 16
                assert voff.min() >= 0 and voff.max() + k_extent <= a_bytes, ("A256", g, r0)
            else:
                if la.swiglu:
                    wnb, within = row // WTN, row % WTN
                    br = (within // (WTN // 2)) * la.N + np.minimum(n0 + wnb * (WTN // 2) + within % (WTN // 2), la.N - 1)
                else:
                    br = np.minimum(n0 + row, la.N - 1)
                voff = br.astype(np.int64) * la.ldb * 2 + chunk * 16
                assert voff.min() >= 0 and b_base + voff.max() + k_extent <= la.b_bytes, ("B256", g, nt)
            assert voff.max() + k_extent - 16 < 1 << 32
            for slot in range(2):
                lds = slot * STAGE256 + (0 if loads_a else 256 * ROW_BYTES) + lrow0 * ROW_BYTES + i * 1024 + lane * 16
                lo_, hi_ = slot * STAGE256 + (0 if loads_a else 256 * ROW_BYTES), slot * STAGE256 + (256 if loads_a else 512) * ROW_BYTES
                assert lds.min() >= lo_ and lds.max() + 16 <= hi_, ("LDS256", wave, i)
    # epilogue
    pitch = bn_out * 2 + 16
    assert 256 * pitch <= PIPE_BYTES
    rows_valid = min(256, row_end - r0)
    assert rows_valid == 256, ("a 256-row chunk", g, r0)
    cols = n0 + np.arange(0, bn_out, 8)
    cols = cols[cols < la.N]
    assert r0 + rows_valid <= la.M
    assert ((r0 + rows_valid - 1) * la.ldc + cols.max()) * 2 + 16 <= la.M * la.ldc * la.c_esize, ("C256", g, r0)
    assert cols[0] == n0 and cols.max() + 8 >= min(n0 + bn_out, la.N)
    written[r0:r0 + rows_valid, nt] += 1


def _check_tile(la, g, row_begin, row_end, r_off, bm, nt, nk, byt, written, lwaves=L_WAVES):
    lane = np.arange(WAVE)
    WM = 1 if bm == 16 else 2
    WN = 8 // WM
    WTN = BN // WN
    bn_out = BN // 2 if la.swiglu else BN
    r0 = row_begin + r_off
    n0 = nt * bn_out
    st = stage_bytes(bm, la.fp4)
    a_instr = bm // ROWS_PER_INSTR
    a_per_wave = cdiv(a_instr, lwaves)
    b_per_wave = BN // ROWS_PER_INSTR // lwaves
    k_extent = (nk - 1) * ROW_BYTES + 16        # bytes a lane reads past its offset over the K loop
    assert st["count"] * st["data"] <= MX_DATA if la.mx else st["count"] * st["bytes"] <= PIPE_BYTES

    a_base = byt(g * la.a_group_stride) if la.uniform_rows else 0
    a_bytes = la.A_rows * byt(la.lda)

    def a_row_of(row):
        r = np.minimum(r0 + row, row_end - 1)
        if la.a_rows is not None:
            ar = la.a_rows[r].astype(np.int64)
        else:
            ar = (r - row_begin if la.uniform_rows else r).astype(np.int64)
        return np.clip(ar, 0, la.A_rows - 1)

    def b_row_of(rho):
        if la.swiglu:
            wnb, within = rho // WTN, rho % WTN
            half, idx = within // (WTN // 2), within % (WTN // 2)
            return half * la.N + np.minimum(n0 + wnb * (WTN // 2) + idx, la.N - 1)
        return np.minimum(n0 + rho, la.N - 1)

    b_base = byt(g * la.b_stride)
    for lw in range(lwaves):
        for i in range(a_per_wave):
            instr = lw + lwaves * i
            if not (a_instr % lwaves == 0 or instr < a_instr):
                continue
            row = instr * ROWS_PER_INSTR + lane // 8
            chunk = (lane % 8) ^ ((row >> 1) & 7)
            voff = a_row_of(row) * byt(la.lda) + chunk * 16
            assert voff.min() >= 0 and a_base + voff.max() + k_extent <= a_bytes, ("A", g, r0, bm)
            assert voff.max() + k_extent - 16 < 1 << 32
            lds = instr * 1024 + lane * 16
            assert lds.max() + 16 <= bm * ROW_BYTES, ("A LDS", bm)
        for i in range(b_per_wave):
            instr = lw * b_per_wave + i
            rho = instr * ROWS_PER_INSTR + lane // 8
            chunk = (lane % 8) ^ ((rho >> 1) & 7)
            voff = b_row_of(rho) * byt(la.ldb) + chunk * 16
            assert voff.min() >= 0 and voff.max() + k_extent - 16 < 1 << 32
            assert b_base + voff.max() + k_extent <= la.b_bytes, ("B", g, nt)
            lds = bm * ROW_BYTES + instr * 1024 + lane * 16
            assert lds.max() + 16 <= st["data"], ("B LDS", bm)
        if la.mx:
            # scale batches: batch b (stages b spb .. b spb + spb - 1) is 16 bytes of every A and
            # B row; piece q of a batch brings rows 16 q .. 16 q + 15 (A rows, then B rows), lane l
            # dword l % 4 of row 16 q + l / 4, clamped to the row's last dword of the K range
            sdw = st["sdw"]
            spb = SC_BATCH_BYTES // (4 * sdw)
            apc = st["scale_rows_a"] // 16
            npc = apc + BN // 16
            sc_per_wave = cdiv(npc, lwaves)
            assert sc_per_wave <= 6 and spb >= 2
            last_dw = nk * sdw - 1
            for u in range(sc_per_wave):
                q = lw + lwaves * u
                if q >= npc:
                    continue
                dws = np.stack([np.minimum(4 * b + lane % 4, last_dw) for b in range(cdiv(nk, spb))])
                assert dws.min() >= 0
                if q < apc:
                    off = a_row_of(q * 16 + lane // 4) * la.lda_scale
                    assert off.max() < 1 << 32
                    assert off.max() + 4 * dws.max() + 4 <= la.A_rows * la.lda_scale, ("A scale", g)
                else:
                    roff = b_row_of((q - apc) * 16 + lane // 4) * la.ldb_scale
                    assert roff.max() < 1 << 32
                    off = g * la.b_scale_stride + roff
                    assert off.max() + 4 * dws.max() + 4 <= la.b_scale_bytes, ("B scale", g)
                for slot in (0, 1):
                    lds = MX_DATA + slot * SC_SLOT + q * SC_PIECE + lane * 4
                    assert lds.min() >= MX_DATA and lds.max() + 4 <= MX_DATA + (slot + 1) * SC_SLOT
            # the rows the MFMA waves read lie inside the slot's A and B parts
            assert bm <= st["scale_rows_a"] and npc * SC_PIECE <= SC_SLOT
    # epilogue: LDS staging of the output tile, then 16-byte stores of valid rows and columns
    pitch = bn_out * la.c_esize + 16
    assert bm * pitch <= PIPE_BYTES, ("epilogue LDS", bm)
    if la.mx:   # staging (twice for the SwiGLU-backward epilogue) below the scale slots
        assert 2 * bm * (BN * 2 + 16) <= MX_DATA, ("epilogue LDS", bm)
    rows_valid = min(bm, row_end - r0)
    assert rows_valid >= 1
    cols_per_chunk = 16 // la.c_esize
    cols = n0 + np.arange(0, bn_out, cols_per_chunk)
    cols = cols[cols < la.N]
    assert r0 + rows_valid <= la.M
    last = ((r0 + rows_valid - 1) * la.ldc + cols.max()) * la.c_esize + 16
    assert last <= la.M * la.ldc * la.c_esize, ("C", g, r0)
    # the chunks' columns are exactly this column tile's part of [0, N)
    assert cols[0] == n0 and cols.max() + cols_per_chunk >= min(n0 + bn_out, la.N)
    written[r0:r0 + rows_valid, nt] += 1
    if la.swiglu and la.aux_ld:
        assert (r0 + rows_valid - 1) * la.aux_ld + la.N + min(n0 + bn_out, la.N) <= la.M * la.aux_ld
