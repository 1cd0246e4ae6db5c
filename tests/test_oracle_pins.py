"""Pins for the CPU oracle (no GPU).

The oracle is trusted only because of these checks, none of which re-uses its
arithmetic: exact bf16 bit patterns, integer invariants of the tile geometry,
a pure-Python brute force on tiny vocabularies (tests/brute.py), closed forms,
finite differences, and float64 library routines (torch.logsumexp,
log_softmax, cross_entropy, autograd).  ``test_pins_catch_planted_mistakes``
builds deliberately broken copies of the oracle and checks that the pins fail.
"""
from __future__ import annotations

import math
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
from tests import brute

IGNORE = -100
LN_151936 = math.log(151936)


# --------------------------------------------------------------------------
# helpers (input construction only; no method arithmetic)
# --------------------------------------------------------------------------
def bf16_bits(values) -> np.ndarray:
    """Round float values to bf16 (torch RNE) and return the bit patterns."""
    t = torch.as_tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def random_bf16(rng: np.random.Generator, shape, sigma=2.0) -> np.ndarray:
    return bf16_bits(rng.normal(0.0, sigma, size=shape))


def decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> float64 via struct (brute path), elementwise."""
    flat = [brute.bf16_bits_to_float(b) for b in bits.reshape(-1)]
    return np.asarray(flat, dtype=np.float64).reshape(bits.shape)


def close(a, b, tol):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape
    with np.errstate(invalid="ignore"):
        both_nan = np.isnan(a) & np.isnan(b)
        same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
        diff = np.abs(a - b)
        ok = both_nan | same_inf | (diff <= tol)
        assert ok.all(), f"max diff {diff[~ok].max()} > {tol}"


# --------------------------------------------------------------------------
# pins, each a function of an oracle instance
# --------------------------------------------------------------------------
def pin_bf16_decode(o):
    known = {0x3F80: 1.0, 0xBF80: -1.0, 0x4049: 3.140625, 0x0000: 0.0, 0x4000: 2.0,
             0x7F80: math.inf, 0xFF80: -math.inf, 0x0001: 2.0 ** -133,
             0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0xC2C8: -100.0}
    for bits, val in known.items():
        assert o.bf16_to_f64(bits) == val, hex(bits)
    assert math.copysign(1.0, o.bf16_to_f64(0x8000)) == -1.0
    assert math.isnan(o.bf16_to_f64(0x7FC0))
    # every pattern against torch's bfloat16 -> float64 conversion
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = np.array([o.bf16_to_f64(int(b)) for b in range(0, 65536, 7)])
    sel = ref[::7]
    assert np.array_equal(np.isnan(got), np.isnan(sel))
    m = ~np.isnan(sel)
    assert np.array_equal(got[m], sel[m])


def pin_geometry(o):
    # the pages' sizes: 64 tiles over 151936 and 152576 columns
    assert set(np.diff(o.tile_bounds(151936, 64))) == {2374}
    assert set(np.diff(o.tile_bounds(152576, 64))) == {2384}
    rng = np.random.default_rng(5)
    cases = [(10, 3), (7, 7), (1, 1), (100, 8), (152576, 63), (151936, 1)]
    cases += [(int(v), int(rng.integers(1, v + 1))) for v in rng.integers(1, 5000, size=40)]
    for v, t in cases:
        b = o.tile_bounds(v, t)
        assert b.shape == (t + 1,)
        assert b[0] == 0 and b[-1] == v  # exact cover, last bound pinned to V
        w = np.diff(b)
        assert (w >= 1).all()  # T <= V: no empty tile
        assert set(w) <= {v // t, -(-v // t)}  # equal as possible
        assert w.sum() == v
    for t in (64, 63, 9, 1):
        for s in sorted({1, 2, 3, 4, 7, 8, t} & set(range(1, t + 1))):
            f = o.shard_tiles(t, s)
            assert f[0] == 0 and f[-1] == t
            assert set(np.diff(f)) <= {t // s, -(-t // s)} and (np.diff(f) >= 1).all()
    assert list(np.diff(o.shard_tiles(64, 4))) == [16] * 4
    # Reading R1/R2 (floor, remainder toward the last tile): where T does not
    # divide V the narrow tiles come first and the last tile is the widest, so
    # the last bound is the one the remainder moves.  Exact values, then a
    # brute-force search of the definition "largest b with b * T <= t * V"
    # (no integer division) on small non-divisible sizes.  A ceiling reading
    # gives [0, 4, 7, 10] and [0, 3, 5, 7] here.
    assert list(o.tile_bounds(10, 3)) == [0, 3, 6, 10]
    assert list(o.tile_bounds(7, 4)) == [0, 1, 3, 5, 7]
    assert list(o.tile_bounds(152577, 64)[:3]) == [0, 2384, 4768]
    assert list(o.shard_tiles(7, 3)) == [0, 2, 4, 7]
    assert list(o.shard_tiles(64, 3)) == [0, 21, 42, 64]

    def largest_multiple_below(t, v, tt):
        b = 0
        while (b + 1) * tt <= t * v:
            b += 1
        return b

    for v, t in [(10, 3), (7, 4), (23, 5), (100, 7), (129, 8), (37, 36), (61, 9)]:
        want = [largest_multiple_below(i, v, t) for i in range(t + 1)]
        assert list(o.tile_bounds(v, t)) == want, (v, t)
        if t >= 2:
            s = max(1, t // 3 + 1)
            want_s = [largest_multiple_below(i, t, s) for i in range(s + 1)]
            assert list(o.shard_tiles(t, s)) == want_s, (t, s)
    for bad in ((0, 1), (5, 0), (5, 6)):
        with pytest.raises(oracle.OracleError):
            o.tile_bounds(*bad)
    with pytest.raises(oracle.OracleError):
        o.shard_tiles(8, 9)


def pin_fwd_brute(o):
    rng = np.random.default_rng(11)
    for v in (1, 2, 3, 5, 8, 17, 64):
        n = 2 * v + 3
        ld = v + 8 + (-v) % 8  # padding and an ld wider than the row
        bits = random_bf16(rng, (n, ld))
        tgt = np.concatenate([np.arange(v), rng.integers(0, v, size=n - v)]).astype(np.int32)
        mask = rng.random(n) < 0.8
        tgt[rng.random(n) < 0.15] = IGNORE
        logp, lse, rc, _ = o.fwd(bits, tgt, mask, real_vocab=v)
        assert rc == 0
        rows = decode(bits[:, :v]).tolist()
        bl, bs = brute.fwd(rows, tgt, mask, v)
        close(logp, bl, 1e-12)
        close(lse, bs, 1e-12)
        # the fp64 entry point on the decoded values agrees bit for bit
        l2, s2, _, _ = o.fwd(decode(bits), tgt, mask, real_vocab=v)
        assert np.array_equal(l2, logp) and np.array_equal(s2, lse)


def pin_closed_forms(o):
    v = 151936
    cs = np.array([0.0, 1.5, -3.0, 7.25])
    x = np.repeat(bf16_bits(cs)[:, None], v, axis=1)
    tgt = np.array([0, 17, v - 1, 75968], dtype=np.int32)
    logp, lse, _, _ = o.fwd(x, tgt, None, real_vocab=v)
    close(lse, cs + LN_151936, 1e-12)
    close(logp, np.full(4, -LN_151936), 1e-12)
    # one finite value a, the rest -inf: LSE == a and logp == 0, exactly
    ninf = bf16_bits([-np.inf])[0]
    for v2, pos, a in ((64, 5, 3.25), (151936, 151935, -7.5), (1, 0, 12.0)):
        row = np.full((1, v2), ninf, dtype=np.uint16)
        row[0, pos] = bf16_bits([a])[0]
        lp, ls, _, _ = o.fwd(row, np.array([pos], np.int32), None, real_vocab=v2)
        assert ls[0] == a and lp[0] == 0.0
        # k equal values: a + ln k
        k = min(v2, 9)
        row[0, :] = ninf
        row[0, :k] = bf16_bits([a])[0]
        _, ls, _, _ = o.fwd(row, np.array([0], np.int32), None, real_vocab=v2)
        close(ls, [a + math.log(k)], 1e-12)
    # shift invariance with integer logits (exact in bf16 up to 256)
    rng = np.random.default_rng(3)
    ints = rng.integers(-64, 65, size=(6, 300)).astype(np.float64)
    t6 = rng.integers(0, 300, size=6).astype(np.int32)
    l0, s0, _, _ = o.fwd(bf16_bits(ints), t6, None, real_vocab=300)
    l1, s1, _, _ = o.fwd(bf16_bits(ints + 64.0), t6, None, real_vocab=300)
    close(l1, l0, 1e-12)
    close(s1 - s0, np.full(6, 64.0), 1e-12)
    # the selected probabilities over every target sum to one
    for v3 in (1, 2, 5, 17):
        row = random_bf16(rng, (1, v3))
        rows = np.repeat(row, v3, axis=0)
        lp, _, _, _ = o.fwd(rows, np.arange(v3, dtype=np.int32), None, real_vocab=v3)
        assert abs(math.fsum(np.exp(lp)) - 1.0) <= 1e-12


def pin_library(o):
    rng = np.random.default_rng(7)
    n, v_real, v_pad, ld = 24, 1000, 1024, 1032
    bits = random_bf16(rng, (n, ld), sigma=3.0)
    bits[:, v_real:] = rng.integers(0, 65536, size=(n, ld - v_real)).astype(np.uint16)
    tgt = rng.integers(0, v_real, size=n).astype(np.int32)
    mask = rng.random(n) < 0.7
    tgt[3] = IGNORE
    logp, lse, _, _ = o.fwd(bits, tgt, mask, real_vocab=v_real)
    xt = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double()[:, :v_real]
    close(lse, torch.logsumexp(xt, dim=1).numpy(), 1e-12)
    act = mask & (tgt != IGNORE)
    ls = torch.log_softmax(xt, dim=1)
    ref = np.where(act, ls[torch.arange(n), torch.from_numpy(np.where(act, tgt, 0)).long()]
                   .numpy(), 0.0)
    close(logp, ref, 1e-12)
    ce_t = torch.from_numpy(np.where(act, tgt, IGNORE)).long()
    ce = torch.nn.functional.cross_entropy(xt, ce_t, ignore_index=IGNORE, reduction="none")
    close(-logp, ce.numpy(), 1e-12)
    assert np.all(logp[~act] == 0.0) and not np.signbit(logp[~act]).any()


def pin_gradient(o):
    rng = np.random.default_rng(13)
    h = 1e-5
    for v in (1, 2, 5, 17):
        n = 5
        x = decode(random_bf16(rng, (n, v)))
        tgt = rng.integers(0, v, size=n).astype(np.int32)
        mask = np.array([1, 1, 0, 1, 1], dtype=bool)
        tgt[4] = IGNORE
        g = rng.normal(size=n)
        _, lse, _, _ = o.fwd(x, tgt, mask, real_vocab=v)
        d = o.bwd(x, tgt, mask, lse, g, real_vocab=v, padded_vocab=v + 3)
        assert d.shape == (n, v + 3) and np.all(d[:, v:] == 0.0)
        fd = np.zeros((n, v))
        for j in range(v):
            xp, xm = x.copy(), x.copy()
            xp[:, j] += h
            xm[:, j] -= h
            lpp, _, _, _ = o.fwd(xp, tgt, mask, real_vocab=v)
            lpm, _, _, _ = o.fwd(xm, tgt, mask, real_vocab=v)
            fd[:, j] = g * (lpp - lpm) / (2 * h)
        close(d[:, :v], fd, 1e-7)
        act = mask & (tgt != IGNORE)
        assert np.all(d[~act] == 0.0)
        assert np.all(np.abs(d.sum(axis=1)) <= 1e-12 * (1 + np.abs(g)))
        # autograd in float64
        xt = torch.from_numpy(x).requires_grad_(True)
        ls = torch.log_softmax(xt, dim=1)
        sel = ls[torch.arange(n), torch.from_numpy(np.where(act, tgt, 0)).long()]
        (sel * torch.from_numpy(np.where(act, g, 0.0))).sum().backward()
        close(d[:, :v], xt.grad.numpy(), 1e-12)
        # brute probabilities
        close(d, brute.bwd(x.tolist(), tgt, mask, g, v, v + 3), 1e-12)


def pin_partials(o):
    rng = np.random.default_rng(17)
    for v_real, v_pad, t in ((5, 5, 2), (3, 8, 4), (100, 128, 8), (64, 64, 64), (17, 24, 5)):
        n = 4
        bits = random_bf16(rng, (n, v_pad))
        bits[1, :] = bf16_bits([-np.inf])[0]  # all -inf row
        bits[:, v_real:] = 0x7FC0  # NaN in padding never counts
        pm, ps = o.tile_partials(bits, real_vocab=v_real, padded_vocab=v_pad, num_tiles=t)
        b = o.tile_bounds(v_pad, t)
        x = decode(bits)
        for r in range(n):
            ref = brute.partials(x[r].tolist(), b.tolist(), v_real)
            close(pm[r], [m for m, _ in ref], 1e-12)
            close(ps[r], [s for _, s in ref], 1e-12)
            for tt, (m, s) in enumerate(ref):
                if m == -math.inf:  # identity partial, exactly
                    assert pm[r, tt] == -math.inf and ps[r, tt] == 0.0
    # the decomposition is an exact regrouping: merging the partials in
    # ascending tile order reproduces the full-row LSE
    n, v = 8, 151936
    bits = random_bf16(rng, (n, v))
    pm, ps = o.tile_partials(bits, real_vocab=v, padded_vocab=v, num_tiles=64)
    _, lse, _, _ = o.fwd(bits, np.zeros(n, np.int32), None, real_vocab=v)
    for r in range(n):
        mm = max(pm[r])
        merged = mm + math.log(math.fsum(s * math.exp(m - mm) for m, s in zip(pm[r], ps[r])))
        assert abs(merged - lse[r]) <= 1e-12


def pin_errors_and_nonfinite(o):
    v, v_pad = 50, 56
    rng = np.random.default_rng(19)
    bits = random_bf16(rng, (6, v_pad))
    tgt = np.array([0, -1, v, v_pad - 1, 3, 4], dtype=np.int32)
    mask = np.array([1, 0, 1, 1, 1, 1], dtype=bool)
    logp, lse, rc, bad = o.fwd(bits, tgt, mask, real_vocab=v, raise_on_error=False)
    assert rc == oracle.ERR_TARGET_RANGE and bad == 2
    assert np.isnan(logp[2]) and np.isnan(logp[3]) and logp[1] == 0.0
    assert np.isfinite(lse).all()
    with pytest.raises(oracle.OracleError):
        o.fwd(bits, tgt, mask, real_vocab=v)
    # non-finite LSE: all -inf row (active -> error, inactive -> fine)
    b2 = random_bf16(rng, (3, v))
    b2[1, :] = bf16_bits([-np.inf])[0]
    _, ls, rc, bad = o.fwd(b2, np.zeros(3, np.int32), None, real_vocab=v, raise_on_error=False)
    assert rc == oracle.ERR_NONFINITE_LSE and bad == 1 and ls[1] == -math.inf
    _, ls, rc, _ = o.fwd(b2, np.zeros(3, np.int32), np.array([1, 0, 1]), real_vocab=v)
    assert rc == 0 and ls[1] == -math.inf
    # NaN or +inf among the real columns: LSE is NaN
    b3 = random_bf16(rng, (3, v))
    b3[0, 7] = 0x7FC0
    b3[1, 9] = bf16_bits([np.inf])[0]
    _, ls, _, _ = o.fwd(b3, np.zeros(3, np.int32), np.zeros(3), real_vocab=v)
    assert np.isnan(ls[0]) and np.isnan(ls[1]) and np.isfinite(ls[2])
    # empty batch
    lp, ls, rc, _ = o.fwd(np.zeros((0, 8), np.uint16), np.zeros(0, np.int32), None, real_vocab=8)
    assert rc == 0 and lp.shape == (0,)


def pin_padding_and_ld(o):
    rng = np.random.default_rng(23)
    n, v_real, v_pad, ld = 5, 37, 40, 48
    clean = random_bf16(rng, (n, ld))
    clean[:, v_real:] = 0
    dirty = clean.copy()
    dirty[:, v_real:] = rng.integers(0, 65536, size=(n, ld - v_real)).astype(np.uint16)
    tgt = rng.integers(0, v_real, size=n).astype(np.int32)
    a = o.fwd(clean, tgt, None, real_vocab=v_real)
    b = o.fwd(dirty, tgt, None, real_vocab=v_real)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # rows are read at stride ld: compare with the compact copy
    compact = np.ascontiguousarray(clean[:, :v_real])
    c = o.fwd(compact, tgt, None, real_vocab=v_real)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])
    g = rng.normal(size=n)
    d1 = o.bwd(dirty, tgt, None, a[1], g, real_vocab=v_real, padded_vocab=v_pad)
    d2 = o.bwd(compact, tgt, None, a[1], g, real_vocab=v_real, padded_vocab=v_pad)
    assert np.array_equal(d1, d2) and np.all(d1[:, v_real:] == 0.0)


def pin_lmhead(o):
    """Fused LM-head logits: z = h . W^T in fp64 over real vocabulary rows."""
    rng = np.random.default_rng(29)
    n, k, v_real, v_pad = 7, 48, 123, 130
    h = random_bf16(rng, (n, k), sigma=1.0)
    w = random_bf16(rng, (v_pad, k), sigma=0.5)
    w[v_real:] = 0x7FC0  # padding rows hold NaN and must never be read
    z = o.lmhead_logits(h, w, real_vocab=v_real)
    ref = decode(h) @ decode(w[:v_real]).T  # float64 library matmul
    assert z.shape == (n, v_real) and np.isfinite(z).all()
    assert np.max(np.abs(z - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
    # a one-hot hidden state selects one column of W, exactly
    e = np.zeros((3, k), dtype=np.uint16)
    for r, col in enumerate((0, 17, k - 1)):
        e[r, col] = bf16_bits([1.0])[0]
    z1 = o.lmhead_logits(e, w, real_vocab=v_real)
    for r, col in enumerate((0, 17, k - 1)):
        assert np.array_equal(z1[r], decode(w[:v_real, col]))
    # the matrix-product form agrees with the plain loops (and so with the decode
    # through struct above), padding rows unread
    zb = o.lmhead_logits_blas(h, w, real_vocab=v_real)
    assert zb.shape == z.shape and np.max(np.abs(zb - z)) <= 1e-12 * max(1.0, np.max(np.abs(z)))
    assert np.array_equal(o.lmhead_logits_blas(e, w, real_vocab=v_real), z1)
    # the selected-token logp of the fused variant is the log-softmax of z
    tgt = rng.integers(0, v_real, size=n).astype(np.int32)
    lp, ls, _, _ = o.lmhead_fwd(h, w, tgt, real_vocab=v_real)
    ls_ref = torch.logsumexp(torch.from_numpy(ref), dim=1).numpy()
    close(ls, ls_ref, 1e-12)
    close(lp, ref[np.arange(n), tgt] - ls_ref, 1e-12)


def pin_entropy(o):
    """H = -sum p log p: brute force, closed forms, a float64 library routine, shift
    invariance, and the bf16 path against the f64 path on decoded values."""
    rng = np.random.default_rng(31)
    for v in (1, 2, 3, 7, 64):
        bits = random_bf16(rng, (4, v))
        x = decode(bits)
        want = [brute.entropy(list(row)) for row in x]
        close(o.entropy(bits, real_vocab=v), want, 1e-12)
        close(o.entropy(x, real_vocab=v), want, 1e-12)
    v = 151936
    x = np.zeros((6, v))
    x[1] = 3.5                      # uniform: H = log V
    x[2] = -np.inf
    x[2, 17] = 2.0                  # one finite value: H = 0
    x[3] = -np.inf
    x[3, [5, 99, 70000]] = -1.25    # three equal finite values: H = log 3
    x[4] = -np.inf                  # no distribution: NaN
    x[5, :2] = [0.0, math.log(3.0)]  # p = (1/4, 3/4) over 2 columns
    x[5, 2:] = -np.inf
    h = o.entropy(x, real_vocab=v)
    close(h[:2], [LN_151936, LN_151936], 1e-9)
    assert h[2] == 0.0
    close(h[3], math.log(3.0), 1e-12)
    assert math.isnan(h[4])
    close(h[5], -(0.25 * math.log(0.25) + 0.75 * math.log(0.75)), 1e-12)
    # float64 library routine and shift invariance
    y = rng.normal(0.0, 3.0, size=(24, 1000))
    lib = torch.distributions.Categorical(logits=torch.from_numpy(y)).entropy().numpy()
    close(o.entropy(y, real_vocab=1000), lib, 1e-10)
    close(o.entropy(y + 40.0, real_vocab=1000), lib, 1e-10)
    # padding and ld: only the real columns count
    z = np.full((3, 48), np.nan)
    z[:, :37] = rng.normal(size=(3, 37))
    close(o.entropy(z, real_vocab=37),
          [brute.entropy(list(row[:37])) for row in z], 1e-12)


def pin_gradient_ex(o):
    """The extended backward against float64 autograd of
    F = sum_r [a_r g_r logp_r + gl_r LSE_r + gh_r H_r], against brute force on tiny
    rows, and against central differences of the oracle's own forward and entropy."""
    rng = np.random.default_rng(37)
    n, v_real, v_pad = 7, 40, 48
    x = rng.normal(0.0, 2.0, size=(n, v_pad))
    x[:, v_real:] = np.nan
    x[2, 3] = -np.inf  # a -inf column: p = 0, 0 log 0 = 0
    tgt = rng.integers(0, v_real, size=n).astype(np.int32)
    tgt[4] = IGNORE
    mask = np.ones(n, dtype=np.uint8)
    mask[1] = 0
    g, gl, gh = rng.normal(size=n), rng.normal(size=n), rng.normal(size=n)
    _, lse, _, _ = o.fwd(x, tgt, mask, real_vocab=v_real)
    ent = o.entropy(x, real_vocab=v_real)
    xt = torch.from_numpy(x[:, :v_real].copy()).requires_grad_(True)
    lsm = torch.log_softmax(xt, dim=1)
    act = torch.from_numpy((mask != 0) & (tgt != IGNORE))
    tsafe = torch.from_numpy(np.where(tgt == IGNORE, 0, tgt).astype(np.int64))
    logp = lsm.gather(1, tsafe[:, None])[:, 0] * act
    p = lsm.exp()
    h = -(p * torch.where(p > 0, lsm, torch.zeros_like(lsm))).sum(1)  # 0 log 0 = 0
    for use_g, use_gl, use_gh in ((1, 0, 0), (0, 1, 0), (0, 0, 1), (1, 1, 1)):
        xt.grad = None
        f = (torch.from_numpy(g) * logp * use_g).sum() + (torch.from_numpy(gl) * torch.logsumexp(
            xt, 1) * use_gl).sum() + (torch.from_numpy(gh) * h * use_gh).sum()
        f.backward(retain_graph=True)
        d = o.bwd_ex(x, tgt, mask, lse, real_vocab=v_real, padded_vocab=v_pad, ent=ent,
                     g=g if use_g else None, g_lse=gl if use_gl else None,
                     g_ent=gh if use_gh else None)
        close(d[:, :v_real], xt.grad.numpy(), 1e-10)
        assert (d[:, v_real:] == 0).all()
    # with only g it is the plain backward
    d0 = o.bwd_ex(x, tgt, mask, lse, real_vocab=v_real, padded_vocab=v_pad, g=g)
    close(d0, o.bwd(x, tgt, mask, lse, g, real_vocab=v_real, padded_vocab=v_pad), 0.0)
    # brute force on tiny bf16 rows
    for v in (2, 5, 9):
        bits = random_bf16(rng, (3, v))
        xb = decode(bits)
        t3 = rng.integers(0, v, size=3).astype(np.int32)
        m3 = np.array([1, 0, 1], dtype=np.uint8)
        g3, gl3, gh3 = rng.normal(size=3), rng.normal(size=3), rng.normal(size=3)
        _, l3, _, _ = o.fwd(bits, t3, m3, real_vocab=v)
        e3 = o.entropy(bits, real_vocab=v)
        got = o.bwd_ex(bits, t3, m3, l3, real_vocab=v, padded_vocab=v + 3, ent=e3, g=g3,
                       g_lse=gl3, g_ent=gh3)
        want = brute.bwd_ex([list(r) for r in xb], t3, m3, g3, gl3, gh3, v, v + 3)
        close(got, want, 1e-12)
    # central differences of the oracle's own LSE and entropy
    eps = 1e-6
    for r, j in ((0, 0), (3, 11), (6, v_real - 1)):
        xp, xm = x.copy(), x.copy()
        xp[r, j] += eps
        xm[r, j] -= eps
        dl = (o.fwd(xp, tgt, mask, real_vocab=v_real)[1][r]
              - o.fwd(xm, tgt, mask, real_vocab=v_real)[1][r]) / (2 * eps)
        dh = (o.entropy(xp, real_vocab=v_real)[r] - o.entropy(xm, real_vocab=v_real)[r]) / (2 * eps)
        one = np.zeros(n)
        one[r] = 1.0
        got_l = o.bwd_ex(x, tgt, mask, lse, real_vocab=v_real, padded_vocab=v_pad, g_lse=one)
        got_h = o.bwd_ex(x, tgt, mask, lse, real_vocab=v_real, padded_vocab=v_pad, ent=ent,
                         g_ent=one)
        close(got_l[r, j], dl, 1e-6)
        close(got_h[r, j], dh, 1e-6)
    # inactive rows get the LSE and entropy terms but no logp term
    d1 = o.bwd_ex(x, tgt, mask, lse, real_vocab=v_real, padded_vocab=v_pad, g=g)
    assert (d1[1] == 0).all() and (d1[4] == 0).all()


def pin_entropy_partials(o):
    rng = np.random.default_rng(41)
    for v_real, v_pad, t in ((5, 5, 2), (3, 8, 4), (100, 128, 8), (17, 24, 5)):
        bits = random_bf16(rng, (3, v_pad))
        bits[1, :2] = 0xFF80  # -inf columns
        x = decode(bits)
        b = o.tile_bounds(v_pad, t)
        _, _, pe = o.tile_partials(bits, real_vocab=v_real, padded_vocab=v_pad, num_tiles=t,
                                   with_entropy=True)
        for r in range(3):
            close(pe[r], brute.entropy_partials(list(x[r]), list(b), v_real), 1e-12)


PINS = [pin_bf16_decode, pin_geometry, pin_fwd_brute, pin_closed_forms, pin_library,
        pin_gradient, pin_partials, pin_errors_and_nonfinite, pin_padding_and_ld, pin_lmhead,
        pin_entropy, pin_gradient_ex, pin_entropy_partials]


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.get()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(orc, pin):
    pin(orc)


# --------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle source must fail some pin
# --------------------------------------------------------------------------
MUTANTS = {
    "dropped_last_term": ("for (int64_t j = 0; j < n; ++j) sum += exp(x[j] - m);",
                          "for (int64_t j = 0; j + 1 < n; ++j) sum += exp(x[j] - m);"),
    "gradient_sign": ("d[j] = g * (onehot - exp(x[j] - lse));",
                      "d[j] = g * (exp(x[j] - lse) - onehot);"),
    "target_off_by_one": ("jb->logp[r] = x[t] - lse;",
                          "jb->logp[r] = x[t > 0 ? t - 1 : t] - lse;"),
    "row_stride_transposed": ("if (jb->xd) return jb->xd + r * jb->ld;\n"
                              "  decode_row(jb->xb + r * jb->ld, n, scratch);",
                              "if (jb->xd) return jb->xd + r * jb->real_vocab;\n"
                              "  decode_row(jb->xb + r * jb->real_vocab, n, scratch);"),
    "mask_ignored": ("int m = mask ? (mask[r] != 0) : 1;", "int m = 1; (void)mask;"),
    "padding_counted": ("if (hi > jb->real_vocab) hi = jb->real_vocab;", ""),
    "bf16_shift": ("uint32_t w = (uint32_t)bits << 16;", "uint32_t w = (uint32_t)bits << 15;"),
    "bounds_truncated": ("bounds[t] = (padded_vocab * (int64_t)t) / (int64_t)num_tiles;",
                         "bounds[t] = (padded_vocab / (int64_t)num_tiles) * (int64_t)t;"),
    "bounds_ceil": ("bounds[t] = (padded_vocab * (int64_t)t) / (int64_t)num_tiles;",
                    "bounds[t] = (padded_vocab * (int64_t)t + num_tiles - 1) / (int64_t)num_tiles;"),
    "shards_ceil": ("first_tile[s] = (int32_t)(((int64_t)s * num_tiles) / num_shards);",
                    "first_tile[s] = (int32_t)(((int64_t)s * num_tiles + num_shards - 1) / "
                    "num_shards);"),
    "onehot_dropped": ("double onehot = (j == (int64_t)t) ? 1.0 : 0.0;",
                       "double onehot = 0.0;"),
    "identity_partial_wrong": ("double m = -INFINITY, s = 0.0, a = 0.0;",
                               "double m = -INFINITY, s = 1.0, a = 0.0;"),
    "lse_unshifted_max": ("return m + log(sum);", "return log(sum);"),
    "lmhead_dropped_k": ("for (int64_t q = 0; q < jb->k; ++q) acc += hr[q] * wr[q];",
                         "for (int64_t q = 0; q + 1 < jb->k; ++q) acc += hr[q] * wr[q];"),
    "lmhead_wrong_hidden_row": ("const double* hr = jb->hd + r * jb->k;",
                                "const double* hr = jb->hd + (r > 0 ? r - 1 : r) * jb->k;"),
    "entropy_sign": ("h -= exp(lp) * lp;", "h += exp(lp) * lp;"),
    "entropy_grad_without_h": ("v -= gh * p * ((x[j] - lse) + h);", "v -= gh * p * (x[j] - lse);"),
    "entropy_grad_sign": ("v -= gh * p * ((x[j] - lse) + h);", "v += gh * p * ((x[j] - lse) + h);"),
    "lse_grad_dropped": ("double v = g * (oh - p) + gl * p;", "double v = g * (oh - p);"),
    "ex_onehot_dropped": ("const double oh = (j == (int64_t)t) ? 1.0 : 0.0;",
                          "const double oh = 0.0;"),
    "ex_logp_term_on_inactive": ("const double g = (act && jb->g) ? jb->g[r] : 0.0;",
                                 "const double g = jb->g ? jb->g[r] : 0.0;"),
    "entropy_partial_unshifted": ("a += exp(x[j] - m) * (x[j] - m);", "a += exp(x[j] - m) * x[j];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(tmp_path: Path, name):
    old, new = MUTANTS[name]
    src = oracle.SOURCE.read_text()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.compile_oracle(mutant_src, tmp_path / f"lib_{name}.so")
    mutant = oracle.Oracle(lib)
    failed = []
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, oracle.OracleError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
