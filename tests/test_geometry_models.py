"""CPU models of the kernels' index arithmetic (no GPU): every column a kernel
counts is counted once, every load stays inside what it may read, every output
slot has one writer.  Each model mirrors the indexing of one kernel, term for
term, and takes its tile and shard bounds from the library's own host geometry
(rlk_logp_tile_geometry), so a change to either side that breaks coverage fails
here before it reaches a GPU.

  * stage 1 (tile_partial): per (lane, slot) the chunk a 16-lane group loads and
    the columns it keeps after masking, for every tile of 310 shapes;
  * the one-launch forward+backward's unit schedule (fwd_bwd_units): which
    geometries take it, and that its dX writes cover every column of the row
    once, for 3,000 shapes;
  * the XCD-local block renumbering: a bijection on every grid size used;
  * the fused LM-head's shard launch loop (lmhead_segments, lmhead_tiles): block
    order, weight rows loaded, segment slots written and the segments each tile
    merges, for 12,938 (vocabulary, tiles, shards) shapes.
"""
from __future__ import annotations

import random

import numpy as np

import vocab_selected_token_amd as rlk

GROUP_LANES = 16
SLOTS = 5
PASS_CHUNKS = SLOTS * GROUP_LANES  # 80 chunks = 640 columns per pass
KBV = 256  # vocabulary rows per LM-head block
KBT = 256  # tokens per LM-head block
GROUP_V = 4  # vocabulary blocks per strip of the LM-head block order


def geometry(padded_vocab: int, tiles: int, shards: int = 1):
    return rlk.rlk_logp_tile_geometry(padded_vocab, tiles, shards)


# --------------------------------------------------------------------------
# stage 1
# --------------------------------------------------------------------------
def stage1_tile(lo: int, hi: int):
    """(chunks loaded, columns kept) by the 16 lanes of one group reducing the
    columns [lo, hi), following tile_partial: the chunk cut by the lower bound on
    lane 0, the one cut by the upper bound on lane 1, then passes of 5 slots per
    lane from the 128-byte line holding the first full chunk; slot k of lane gl in
    pass p is chunk base0 + 80 p + 16 k + gl, loaded from an address clamped into
    the full chunks and masked when outside them."""
    loads, cols = [], []
    cf_lo = (lo + 7) >> 3
    cf_hi = max(hi >> 3, cf_lo)
    base0 = cf_lo & ~7
    npass = (cf_hi - base0 + PASS_CHUNKS - 1) // PASS_CHUNKS if cf_hi > cf_lo else 0
    for gl in (0, 1):
        if gl == 0 and hi > lo and (lo & 7):
            c, e_lo, e_hi = lo >> 3, lo & 7, min(hi - ((lo >> 3) << 3), 8)
        elif gl == 1 and hi > lo and (hi & 7) and (hi >> 3) >= cf_lo:
            c, e_lo, e_hi = hi >> 3, 0, hi & 7
        else:
            continue
        loads.append(np.array([c]))
        cols.append(np.arange(c * 8 + e_lo, c * 8 + e_hi))
    if npass:
        p = np.arange(npass)[:, None, None]
        k = np.arange(SLOTS)[None, :, None]
        gl = np.arange(GROUP_LANES)[None, None, :]
        c = (base0 + p * PASS_CHUNKS + k * GROUP_LANES + gl).ravel()
        loads.append(np.clip(c, cf_lo, cf_hi - 1))
        kept = c[(c >= cf_lo) & (c < cf_hi)]
        cols.append((kept[:, None] * 8 + np.arange(8)[None, :]).ravel())
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, dtype=np.int64)
    return cat(loads), cat(cols)


def check_stage1_shape(real: int, pad: int, ld: int, tiles: int):
    bounds, _ = geometry(pad, tiles)
    seen = np.zeros(real, dtype=np.int64)
    for t in range(tiles):
        lo, hi = int(bounds[t]), min(int(bounds[t + 1]), real)
        hi = max(hi, lo)
        loads, cols = stage1_tile(lo, hi)
        if hi == lo:
            assert cols.size == 0 and loads.size == 0  # the identity partial reads nothing
            continue
        # every load inside the row, and inside the chunks that hold the tile
        assert loads.min() >= lo >> 3 and loads.max() < (hi + 7) >> 3, (real, pad, tiles, t)
        assert loads.max() < ld // 8
        # the kept columns are exactly [lo, hi), once each
        assert cols.size == hi - lo and cols.min() == lo and cols.max() == hi - 1, (real, tiles, t)
        np.add.at(seen, cols, 1)
    assert (seen == 1).all(), (real, pad, tiles)


def stage1_shapes():
    rng = random.Random(20261203)
    shapes = [(151936, 151936, 151936, 64), (151936, 152576, 152576, 64),
              (151936, 152576, 152584, 64), (1, 8, 8, 1), (100, 128, 128, 8),
              (2374 * 3 + 1, 2374 * 3 + 8, 2374 * 3 + 8, 3), (9000, 9000, 9000, 65),
              (5000, 5120, 5128, 64), (7, 7, 8, 7), (3001, 3008, 3008, 5)]
    while len(shapes) < 310:
        real = rng.choice([rng.randint(1, 64), rng.randint(1, 5000), rng.randint(1, 200000)])
        pad = real + rng.choice([0, 0, 1, 7, 8, 640, rng.randint(0, 2000)])
        ld = (pad + 7) // 8 * 8 + rng.choice([0, 0, 8, 64])
        tiles = rng.randint(1, min(pad, rng.choice([8, 64, 1024])))
        shapes.append((real, pad, ld, tiles))
    return shapes


def test_stage1_lane_coverage():
    shapes = stage1_shapes()
    assert len(shapes) == 310
    for real, pad, ld, tiles in shapes:
        check_stage1_shape(real, pad, ld, tiles)


def test_stage1_model_catches_a_coverage_mistake():
    """The model itself: a pass that started one chunk late would drop a column."""
    loads, cols = stage1_tile(2374, 4748)
    assert np.array_equal(np.sort(cols), np.arange(2374, 4748))
    lo, hi = 2374, 4748
    cf_lo = (lo + 7) >> 3
    assert cf_lo & 7  # this tile's first full chunk is mid-line: the passes start before it
    _, good = stage1_tile(lo, hi)
    _, shifted = stage1_tile(lo + 8, hi)
    assert set(good.tolist()) - set(shifted.tolist())


# --------------------------------------------------------------------------
# the unit schedule of the one-launch forward+backward
# --------------------------------------------------------------------------
UNIT_MAX_PASS = 4


def fb_desc(real: int, pad: int, tiles: int, n: int = 2):
    return rlk.make_desc(n, real, pad, (pad + 7) // 8 * 8, tiles, 1, -100, False)


def units_fit(real: int, pad: int, tiles: int) -> bool:
    """The rule fwd_bwd_units_fit states: T <= 64, tiles of at least 8 columns,
    and every tile's full chunks within 4 passes of one 16-lane group."""
    if tiles > 64 or pad // tiles < 8:
        return False
    bounds, _ = geometry(pad, tiles)
    for t in range(tiles):
        lo = int(bounds[t])
        hi = max(min(int(bounds[t + 1]), real), lo)
        cf_lo = (lo + 7) >> 3
        cf_hi = max(hi >> 3, cf_lo)
        base0 = cf_lo & ~7
        npass = (cf_hi - base0 + PASS_CHUNKS - 1) // PASS_CHUNKS if cf_hi > cf_lo else 0
        if npass > UNIT_MAX_PASS:
            return False
    return True


def units_dx_chunks(real: int, pad: int, tiles: int):
    """The dX chunks each tile's group writes in fwd_bwd_units: the full chunks of
    its passes (from registers), lane 1's tail chunk (the chunk cut by the tile's
    real upper bound, when the tile has one), and zeros for the chunks whose first
    column lies in the tile's padded bounds at or past V_real."""
    bounds, _ = geometry(pad, tiles)
    out = []
    for t in range(tiles):
        plo, phi = int(bounds[t]), int(bounds[t + 1])
        lo = plo
        hi = max(min(phi, real), lo)
        cf_lo = (lo + 7) >> 3
        cf_hi = max(hi >> 3, cf_lo)
        out.extend(range(cf_lo, cf_hi))
        if hi > lo and (hi & 7) and (hi >> 3) >= cf_lo:
            out.append(hi >> 3)
        out.extend(range(max((plo + 7) >> 3, (real + 7) >> 3), (phi + 7) >> 3))
    return np.array(out, dtype=np.int64)


def unit_shapes():
    rng = random.Random(20261204)
    shapes = [(151936, 152576, 64), (151936, 151936, 64), (151936, 152584, 64),
              (8, 8, 1), (63, 64, 8), (64, 64, 8), (65, 72, 9), (2504, 2504, 1),
              (2505, 2512, 1), (5000, 5120, 64), (3001, 3008, 5), (12345, 12352, 7),
              (60, 63, 9), (7, 7, 1), (500, 512, 65)]
    while len(shapes) < 3000:
        tiles = rng.randint(1, rng.choice([4, 64, 80]))
        width = rng.choice([8, 9, 15, 16, rng.randint(8, 64), rng.randint(8, 2600)])
        pad = tiles * width + rng.randint(0, tiles - 1)
        real = max(1, pad - rng.choice([0, 0, 1, 7, 8, 9, rng.randint(0, 3 * width)]))
        shapes.append((real, pad, tiles))
    return shapes


def test_unit_schedule_writes_every_dx_column_once():
    taken = 0
    for real, pad, tiles in unit_shapes():
        fits = units_fit(real, pad, tiles)
        ws = rlk.rlk_logp_fwd_bwd_workspace_bytes(fb_desc(real, pad, tiles, n=3))
        # the library takes the unit schedule exactly where the rule says
        assert ws == (256 + 3 * tiles * 8 if fits else 256), (real, pad, tiles)
        if not fits:
            continue
        taken += 1
        chunks = units_dx_chunks(real, pad, tiles)
        count = np.bincount(chunks, minlength=(pad + 7) // 8)
        assert count.size == (pad + 7) // 8, (real, pad, tiles)  # nothing past the row
        assert (count == 1).all(), (real, pad, tiles, np.flatnonzero(count != 1)[:8])
    assert taken > 2000


def test_unit_model_catches_a_double_write():
    """The model itself: without the tail-chunk rule a tile bound that is not a
    multiple of 8 leaves its chunk unwritten; with the head chunk written as well
    it is written twice."""
    real, pad, tiles = 3001, 3008, 5  # bounds at 601, 1203, ...: not multiples of 8
    chunks = units_dx_chunks(real, pad, tiles)
    assert (np.bincount(chunks) == 1).all()
    bounds, _ = geometry(pad, tiles)
    heads = [int(b) >> 3 for b in bounds[1:-1] if int(b) & 7]
    assert heads
    assert (np.bincount(np.concatenate([chunks, heads])) == 2).any()


# --------------------------------------------------------------------------
# the XCD-local renumbering of blocks
# --------------------------------------------------------------------------
def xcd_local_block(b, nb):
    per, rem, x, l = nb // 8, nb % 8, b % 8, b // 8
    return x * per + np.minimum(x, rem) + l


def test_xcd_local_block_is_a_bijection():
    for nb in list(range(1, 300)) + [511, 512, 513, 4095, 8192, 9536, 131072, 1 << 20]:
        b = np.arange(nb, dtype=np.int64)
        m = xcd_local_block(b, nb)
        assert np.array_equal(np.sort(m), b), nb
        # consecutive work indices share an XCD (block b runs on XCD b % 8)
        if nb >= 16:
            owner = np.empty(nb, dtype=np.int64)
            owner[m] = b % 8
            assert (np.diff(owner) != 0).sum() <= 7


# --------------------------------------------------------------------------
# the fused LM-head's shard launch loop
# --------------------------------------------------------------------------
def inner_tile_bound(v0: int, pad: int, tiles: int) -> int:
    t = ((v0 + 1) * tiles - 1) // pad
    b = ((t + 1) * pad) // tiles
    return b if v0 < b < v0 + KBV else v0 + KBV


def check_lmhead_shape(real: int, pad: int, tiles: int, shards: int, n_tokens: int = 300):
    bounds, first = geometry(pad, tiles, shards)
    bounds = [int(b) for b in bounds]
    n_vb = (real + KBV - 1) // KBV
    n_tb = (n_tokens + KBT - 1) // KBT
    writes = {}  # (vb, slot) -> [(shard, (row_a, row_b))]
    for s in range(shards):
        ta, tb = int(first[s]), int(first[s + 1])
        col_lo, col_hi = bounds[ta], bounds[tb]
        row_lo, row_hi = col_lo, min(col_hi, real)
        if col_lo >= row_hi:
            continue  # a shard of padding only launches no GEMM block
        vb_begin = col_lo // KBV
        n_vbs = (row_hi - 1) // KBV + 1 - vb_begin
        assert 0 <= vb_begin and vb_begin + n_vbs <= n_vb
        # block order: every (vocabulary block, token block) exactly once
        blk = np.arange(n_vbs * n_tb)
        strip = blk // (GROUP_V * n_tb)
        r_in = blk - strip * GROUP_V * n_tb
        strip_w = np.minimum(GROUP_V, n_vbs - strip * GROUP_V)
        vb = vb_begin + strip * GROUP_V + r_in % strip_w
        tb_ = r_in // strip_w
        pairs = set(zip(vb.tolist(), tb_.tolist()))
        assert len(pairs) == n_vbs * n_tb and min(vb) == vb_begin
        assert max(vb) == vb_begin + n_vbs - 1 and max(tb_) == n_tb - 1
        for v in range(vb_begin, vb_begin + n_vbs):
            v0 = v * KBV
            # weight rows loaded: clamped into the shard's real rows
            lo_row = min(max(v0, row_lo), row_hi - 1)
            hi_row = min(max(v0 + KBV - 1, row_lo), row_hi - 1)
            assert row_lo <= lo_row <= hi_row < row_hi <= real
            bnd = inner_tile_bound(v0, pad, tiles)
            inside = [b for b in bounds if v0 < b < v0 + KBV]
            assert len(inside) <= 1 and bnd == (inside[0] if inside else v0 + KBV)
            seg0 = (max(v0, row_lo), min(bnd, v0 + KBV, row_hi))
            seg1 = (max(bnd, row_lo), min(v0 + KBV, row_hi)) if bnd < v0 + KBV else (0, 0)
            c_slot1 = bnd if bnd < v0 + KBV else v0
            if col_lo <= v0 < col_hi:
                writes.setdefault((v, 0), []).append((s, seg0))
            if col_lo <= c_slot1 < col_hi:
                writes.setdefault((v, 1), []).append((s, seg1))
    for k, v in writes.items():
        assert len(v) == 1, (real, pad, tiles, shards, k, v)  # one writer per slot
    # each tile merges its segments, in ascending columns, exactly over its real columns
    for t in range(tiles):
        c0, c1 = bounds[t], bounds[t + 1]
        if c0 >= real:
            continue  # the identity partial, nothing read
        vf = c0 // KBV
        vl = min((min(c1, real) - 1) // KBV, n_vb - 1)
        at = c0
        for v in range(vf, vl + 1):
            slot = 1 if (v == vf and c0 > vf * KBV) else 0
            assert (v, slot) in writes, (real, pad, tiles, shards, t, v, slot)
            a, b = writes[(v, slot)][0][1]
            if b > a:
                assert a == at, (real, pad, tiles, shards, t, v)
                at = b
        assert at == min(c1, real), (real, pad, tiles, shards, t)


def lmhead_shapes():
    rng = random.Random(1)
    out = []
    for _ in range(3000):
        pad = rng.randint(256, 20000)
        real = rng.randint(1, pad)
        tiles = rng.randint(1, pad // 256)
        for s in sorted({1, 2, 3, tiles, rng.randint(1, tiles)} & set(range(1, tiles + 1))):
            out.append((real, pad, tiles, s))
    for real, pad, tiles in [(151936, 152576, 64), (151936, 151936, 64), (700, 4096, 16),
                             (5000, 5120, 16), (2900, 3000, 7), (18500, 19072, 8)]:
        out += [(real, pad, tiles, s) for s in range(1, tiles + 1)]
    return out


def test_lmhead_shard_segments():
    shapes = lmhead_shapes()
    assert len(shapes) == 12938
    for real, pad, tiles, s in shapes:
        check_lmhead_shape(real, pad, tiles, s)
