"""Pure-Python brute force for tiny vocabularies (pins the C oracle).

It deliberately takes a different route from the oracle:
  * bf16 bit patterns are decoded with ``struct`` (not the oracle's decode);
  * the normaliser is the exactly rounded sum ``math.fsum(exp(x_j))`` with no
    max shift (valid for the small |x| the pin tests use);
  * logp is ``log(p_target)`` with ``p_j = exp(x_j) / Z``, not ``x_t - LSE``;
  * the gradient is ``g * (onehot - p)`` from those probabilities.
Only the semantics are shared (which rows count, padding never counts, the
(-inf, 0) identity of an empty tile), and those are stated on the pages.
"""
from __future__ import annotations

import math
import struct


def bf16_bits_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def normaliser(xs) -> float:
    """Z = sum_j exp(x_j), exactly rounded; -inf entries contribute 0."""
    return math.fsum(0.0 if x == -math.inf else math.exp(x) for x in xs)


def lse(xs) -> float:
    z = normaliser(xs)
    return -math.inf if z == 0.0 else math.log(z)


def probs(xs):
    z = normaliser(xs)
    return [(0.0 if x == -math.inf else math.exp(x)) / z for x in xs]


def active(mask, tgt, r, ignore_index) -> bool:
    return (mask is None or bool(mask[r])) and int(tgt[r]) != ignore_index


def fwd(rows, tgt, mask, real_vocab, ignore_index=-100):
    """rows: list of lists of floats (at least real_vocab long). Returns (logp, lse)."""
    out_logp, out_lse = [], []
    for r, row in enumerate(rows):
        xs = list(row[:real_vocab])
        out_lse.append(lse(xs))
        if not active(mask, tgt, r, ignore_index):
            out_logp.append(0.0)
            continue
        p = probs(xs)[int(tgt[r])]
        out_logp.append(math.log(p) if p > 0 else -math.inf)
    return out_logp, out_lse


def bwd(rows, tgt, mask, g, real_vocab, padded_vocab, ignore_index=-100):
    out = []
    for r, row in enumerate(rows):
        d = [0.0] * padded_vocab
        if active(mask, tgt, r, ignore_index):
            p = probs(list(row[:real_vocab]))
            for j in range(real_vocab):
                d[j] = g[r] * ((1.0 if j == int(tgt[r]) else 0.0) - p[j])
        out.append(d)
    return out


def partials(row, bounds, real_vocab):
    """Per-tile (max, sumexp) with max-shifted exactly rounded sums."""
    out = []
    for t in range(len(bounds) - 1):
        xs = list(row[bounds[t]:min(bounds[t + 1], real_vocab)])
        m = max(xs) if xs else -math.inf
        if m == -math.inf:
            out.append((-math.inf, 0.0))
        else:
            out.append((m, math.fsum(math.exp(x - m) for x in xs)))
    return out


def entropy(xs) -> float:
    """H = -sum p log p with exactly rounded sums; p = 0 terms contribute 0."""
    z = normaliser(xs)
    if z == 0.0:
        return math.nan
    terms = []
    for x in xs:
        if x == -math.inf:
            continue
        p = math.exp(x) / z
        if p > 0.0:
            terms.append(-p * math.log(p))
    return math.fsum(terms)


def bwd_ex(rows, tgt, mask, g, g_lse, g_ent, real_vocab, padded_vocab, ignore_index=-100):
    """d = a g (onehot - p) + g_lse p - g_ent p (log p + H); g, g_lse, g_ent may be None."""
    out = []
    for r, row in enumerate(rows):
        d = [0.0] * padded_vocab
        xs = list(row[:real_vocab])
        act = active(mask, tgt, r, ignore_index)
        gr = g[r] if (g is not None and act) else 0.0
        gl = g_lse[r] if g_lse is not None else 0.0
        gh = g_ent[r] if g_ent is not None else 0.0
        if act or gl != 0.0 or gh != 0.0:
            p = probs(xs)
            h = entropy(xs)
            for j in range(real_vocab):
                oh = 1.0 if (act and j == int(tgt[r])) else 0.0
                v = gr * (oh - p[j]) + gl * p[j]
                if gh != 0.0 and p[j] > 0.0:
                    v -= gh * p[j] * (math.log(p[j]) + h)
                d[j] = v
        out.append(d)
    return out


def entropy_partials(row, bounds, real_vocab):
    """Per-tile sum of exp(x - m) (x - m) over the tile's finite real columns."""
    out = []
    for t in range(len(bounds) - 1):
        xs = [x for x in row[bounds[t]:min(bounds[t + 1], real_vocab)] if x != -math.inf]
        if not xs:
            out.append(0.0)
            continue
        m = max(xs)
        out.append(math.fsum(math.exp(x - m) * (x - m) for x in xs))
    return out
