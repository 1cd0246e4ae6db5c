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
