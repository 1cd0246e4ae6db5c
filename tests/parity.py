"""Comparison helpers for GPU-vs-oracle parity (test infrastructure).

Acceptance bar (stated with the reasons in the design notes):
  * LSE on every row and logp on effective-active rows: |gpu - oracle| <= 1e-4;
    non-finite values must match in kind (-inf vs NaN);
  * rows that are not effective-active: logp is +0.0 bit for bit and the whole
    dlogits row is +0.0 bit for bit; padded dlogits columns are +0.0;
  * fp32 dlogits: |gpu - oracle| <= 1e-5;
  * bf16 dlogits: |gpu - oracle| <= 8e-3, or gpu is one of the two bf16 values
    that bracket the oracle value (|gpu - oracle| <= the bf16 spacing there).
"""
from __future__ import annotations

import numpy as np
import torch

TOL_LSE = 1e-4
TOL_LOGP = 1e-4
TOL_D32 = 1e-5
TOL_D16 = 8e-3


def f32_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dlogits_host(d: torch.Tensor) -> np.ndarray:
    """GPU dlogits (fp32 or bf16) as float64 on the host."""
    if d.dtype == torch.bfloat16:
        return bf16_to_f64(d.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return d.double().cpu().numpy()


def effective_active(tgt: np.ndarray, mask: np.ndarray | None, ignore_index: int = -100):
    act = np.ones(tgt.shape[0], dtype=bool) if mask is None else mask.astype(bool)
    return act & (tgt != ignore_index)


def _same_kind(g: np.ndarray, o: np.ndarray) -> np.ndarray:
    return (np.isnan(g) & np.isnan(o)) | (np.isinf(g) & np.isinf(o) & (np.sign(g) == np.sign(o)))


def check_fwd(logp_g, lse_g, logp_o, lse_o, active, tag=""):
    logp_g = np.asarray(logp_g, dtype=np.float32)
    lse_g = np.asarray(lse_g, dtype=np.float32)
    lg, sg = logp_g.astype(np.float64), lse_g.astype(np.float64)
    with np.errstate(invalid="ignore"):
        fin = np.isfinite(lse_o)
        assert np.array_equal(np.isfinite(sg), fin), f"{tag}: LSE finiteness differs"
        assert _same_kind(sg[~fin], lse_o[~fin]).all(), f"{tag}: non-finite LSE kind differs"
        e = np.abs(sg[fin] - lse_o[fin])
        assert e.size == 0 or e.max() <= TOL_LSE, f"{tag}: LSE max err {e.max():.3e}"
        a = active & np.isfinite(logp_o)
        e = np.abs(lg[a] - logp_o[a])
        assert e.size == 0 or e.max() <= TOL_LOGP, f"{tag}: logp max err {e.max():.3e}"
        na = active & ~np.isfinite(logp_o)
        assert _same_kind(lg[na], logp_o[na]).all(), f"{tag}: non-finite logp kind differs"
    # inactive rows: +0.0 exactly
    assert (f32_bits(logp_g[~active]) == 0).all(), f"{tag}: inactive logp not +0.0"
    return {"lse_max_abs": float(np.abs(sg[fin] - lse_o[fin]).max(initial=0.0)),
            "logp_max_abs": float(np.abs(lg[active & np.isfinite(logp_o)]
                                         - logp_o[active & np.isfinite(logp_o)]).max(initial=0.0))}


def bf16_spacing(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.ldexp(1.0, (e - 7).astype(np.int64)), 2.0 ** -133)


def check_bwd(d_g: np.ndarray, d_o: np.ndarray, active: np.ndarray, real_vocab: int,
              bf16: bool, tag="", raw: np.ndarray | None = None):
    """d_g: GPU dlogits as float64 [rows, V_pad]; raw: the GPU bits (for +0.0 checks)."""
    assert d_g.shape == d_o.shape
    bits = raw if raw is not None else None
    # inactive rows and padded columns are +0 exactly (bit patterns all zero)
    if bits is not None:
        assert (bits[~active] == 0).all(), f"{tag}: inactive dlogits row not +0"
        assert (bits[:, real_vocab:] == 0).all(), f"{tag}: padded dlogits column not +0"
    else:
        assert (d_g[~active] == 0).all() and (d_g[:, real_vocab:] == 0).all()
    a = active
    with np.errstate(invalid="ignore"):
        err = np.abs(d_g[a] - d_o[a])
        if bf16:
            allowed = np.maximum(TOL_D16, bf16_spacing(d_o[a]))
            bad = ~(err <= allowed)
        else:
            bad = ~(err <= TOL_D32)
        assert not bad.any(), f"{tag}: dlogits max err {np.nanmax(err):.3e} at {np.argwhere(bad)[:3]}"
    return float(err.max(initial=0.0))


TOL_ENT = 1e-4


def check_entropy(ent_g, ent_o, tag=""):
    """Entropy on every row: |gpu - oracle| <= 1e-4; NaN exactly where the oracle has NaN."""
    eg = np.asarray(ent_g, dtype=np.float32).astype(np.float64)
    eo = np.asarray(ent_o, dtype=np.float64)
    assert np.array_equal(np.isnan(eg), np.isnan(eo)), f"{tag}: entropy NaN rows differ"
    fin = ~np.isnan(eo)
    e = np.abs(eg[fin] - eo[fin])
    assert e.size == 0 or e.max() <= TOL_ENT, f"{tag}: entropy max err {e.max():.3e}"
    return float(e.max(initial=0.0))


def check_bwd_ex(d_g: np.ndarray, d_o: np.ndarray, zero_rows: np.ndarray, real_vocab: int,
                 bf16: bool, tag="", raw: np.ndarray | None = None):
    """The extended backward: rows no term reaches and padded columns are +0 bit for
    bit; every other element within the dlogits tolerance, NaN where the oracle has
    NaN (a bad target)."""
    assert d_g.shape == d_o.shape
    if raw is not None:
        assert (raw[zero_rows] == 0).all(), f"{tag}: unreached dlogits row not +0"
        assert (raw[:, real_vocab:] == 0).all(), f"{tag}: padded dlogits column not +0"
    rows = ~zero_rows
    g, o = d_g[rows], d_o[rows]
    with np.errstate(invalid="ignore"):
        assert np.array_equal(np.isnan(g), np.isnan(o)), f"{tag}: NaN pattern differs"
        fin = ~np.isnan(o)
        err = np.abs(g[fin] - o[fin])
        if bf16:
            bad = ~(err <= np.maximum(TOL_D16, bf16_spacing(o[fin])))
        else:
            bad = ~(err <= TOL_D32)
        assert not bad.any(), f"{tag}: dlogits max err {np.nanmax(err):.3e}"
    return float(err.max(initial=0.0))


# --------------------------------------------------------------------------
# Full-size parity, streamed over row blocks
# --------------------------------------------------------------------------
def host_threads() -> int:
    """Host threads for the oracle and the comparisons: every core this process may
    run on, capped by OMP_NUM_THREADS when the environment sets it (the CPU share a
    shared machine grants one job)."""
    import os
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _check_dx_rows(raw: np.ndarray, d_o: np.ndarray, zero_rows: np.ndarray, real_vocab: int,
                   bf16: bool) -> tuple[int, float]:
    """One sub-block of a large dlogits comparison; raw = GPU bits [rows, V_pad].
    Returns (violations, max abs error over finite elements)."""
    bad = 0
    if zero_rows.any():
        bad += int((raw[zero_rows] != 0).sum())
    bad += int((raw[:, real_vocab:] != 0).sum())
    rows = ~zero_rows
    if not rows.any():
        return bad, 0.0
    if bf16:
        g = (raw[rows, :real_vocab].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        g = raw[rows, :real_vocab].view(np.float32).astype(np.float64)
    o = d_o[rows, :real_vocab]
    with np.errstate(invalid="ignore"):
        gn, on = np.isnan(g), np.isnan(o)
        bad += int((gn != on).sum())
        err = np.abs(g - o)
        err[gn & on] = 0.0
        tol = TOL_D16 if bf16 else TOL_D32
        over = ~(err <= tol)
        if bf16 and over.any():  # R13: a bracketing bf16 neighbour also passes
            idx = np.nonzero(over)
            over[idx] = ~(err[idx] <= bf16_spacing(o[idx]))
        bad += int(over.sum())
        fin = np.isfinite(err)
        return bad, float(err[fin].max(initial=0.0))


def check_dx_block(d_g_raw: np.ndarray, d_o: np.ndarray, zero_rows: np.ndarray, real_vocab: int,
                   bf16: bool, tag: str = "", threads: int | None = None) -> float:
    """check_bwd / check_bwd_ex for large blocks: the same bar, split over host threads
    (numpy releases the interpreter lock inside its loops)."""
    from concurrent.futures import ThreadPoolExecutor
    assert d_g_raw.shape == d_o.shape, (d_g_raw.shape, d_o.shape)
    n = d_g_raw.shape[0]
    step = max(1, -(-n // (threads or host_threads())))
    parts = [(r, min(n, r + step)) for r in range(0, n, step)]
    with ThreadPoolExecutor(max_workers=len(parts)) as ex:
        res = list(ex.map(lambda p: _check_dx_rows(d_g_raw[p[0]:p[1]], d_o[p[0]:p[1]],
                                                   zero_rows[p[0]:p[1]], real_vocab, bf16),
                          parts))
    bad = sum(r[0] for r in res)
    worst = max((r[1] for r in res), default=0.0)
    assert bad == 0, f"{tag}: {bad} dlogits elements off the bar (max err {worst:.3e})"
    return worst


def stream_parity(orc, inp, logp, lse, *, d=None, ent=None, g_lse=None, g_ent=None,
                  block: int = 1024, tag: str = "") -> dict:
    """Every row of a (possibly benchmark-sized) workload against the oracle, streamed
    in blocks of `block` rows so that host memory stays bounded.

    logp, lse   GPU outputs [N] (checked on every row: LSE everywhere, logp on
                effective-active rows, +0.0 elsewhere).
    ent         GPU entropy [N] or None (checked on every row when given).
    d           GPU dlogits [N, >= V_pad] (fp32 or bf16) or None.  Without g_lse
                and g_ent it is the plain backward (g = inp.grad); with either, the
                extended backward (g = inp.grad, g_lse, g_ent; g_ent needs ent).
    The oracle's side uses only the oracle's own LSE and entropy, never the GPU's."""
    import torch
    wl = inp.wl
    n = wl.num_tokens
    thr = host_threads()
    ext = g_lse is not None or g_ent is not None
    logp_h = logp.detach().float().cpu().numpy()
    lse_h = lse.detach().float().cpu().numpy()
    ent_h = None if ent is None else ent.detach().float().cpu().numpy()
    gl_h = None if g_lse is None else g_lse.detach().double().cpu().numpy()
    gh_h = None if g_ent is None else g_ent.detach().double().cpu().numpy()
    tgt_all = inp.targets.cpu().numpy()
    mask_all = inp.mask.cpu().numpy()
    g_all = inp.grad.double().cpu().numpy()
    stats = {"lse_max_abs": 0.0, "logp_max_abs": 0.0, "rows": n}
    if ent is not None:
        stats["entropy_max_abs"] = 0.0
    if d is not None:
        stats["dlogits_max_abs"] = 0.0
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        bits = inp.logits[r0:r1].view(torch.int16).cpu().numpy().view(np.uint16)
        tgt, mask, g = tgt_all[r0:r1], mask_all[r0:r1], g_all[r0:r1]
        act = effective_active(tgt, mask)
        lo, so, _, _ = orc.fwd(bits, tgt, mask, real_vocab=wl.real_vocab, nthreads=thr,
                               raise_on_error=False)
        s = check_fwd(logp_h[r0:r1], lse_h[r0:r1], lo, so, act, f"{tag} rows {r0}:{r1}")
        stats["lse_max_abs"] = max(stats["lse_max_abs"], s["lse_max_abs"])
        stats["logp_max_abs"] = max(stats["logp_max_abs"], s["logp_max_abs"])
        eo = None
        if ent is not None or g_ent is not None:
            eo = orc.entropy(bits, real_vocab=wl.real_vocab, nthreads=thr)
        if ent is not None:
            e = check_entropy(ent_h[r0:r1], eo, f"{tag} rows {r0}:{r1}")
            stats["entropy_max_abs"] = max(stats["entropy_max_abs"], e)
        if d is None:
            continue
        raw_t = d[r0:r1, :wl.padded_vocab].contiguous()
        bf16 = raw_t.dtype == torch.bfloat16
        raw = raw_t.view(torch.int16 if bf16 else torch.int32).cpu().numpy()
        raw = raw.view(np.uint16 if bf16 else np.uint32)
        del raw_t
        if ext:
            do = orc.bwd_ex(bits, tgt, mask, so, real_vocab=wl.real_vocab,
                            padded_vocab=wl.padded_vocab, ent=eo, g=g,
                            g_lse=None if gl_h is None else gl_h[r0:r1],
                            g_ent=None if gh_h is None else gh_h[r0:r1], nthreads=thr,
                            raise_on_error=False)
            zero = np.zeros(r1 - r0, dtype=bool)
        else:
            do = orc.bwd(bits, tgt, mask, so, g, real_vocab=wl.real_vocab,
                         padded_vocab=wl.padded_vocab, nthreads=thr, raise_on_error=False)
            zero = ~act
        w = check_dx_block(raw, do, zero, wl.real_vocab, bf16, f"{tag} dX rows {r0}:{r1}", thr)
        stats["dlogits_max_abs"] = max(stats["dlogits_max_abs"], w)
        del do, raw, bits
    return stats
