"""The comparison helpers themselves (no GPU): the streamed full-size checks must
pass on outputs that meet the bar and fail on each kind of miss.  The "GPU"
outputs here are the oracle's own values rounded to the output precision, with
mistakes planted in them."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import parity as P


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def test_check_dx_block_bar():
    rng = np.random.default_rng(1)
    o = rng.normal(0, 1e-3, size=(40, 96))
    o[:, 90:] = 0.0  # padded columns
    o[3, 5] = 3.3  # a large target-column value: bf16 spacing there is 2^-6
    zero = np.zeros(40, dtype=bool)
    zero[7] = True
    o[7] = 0.0
    raw = _bf16_bits(o)
    assert P.check_dx_block(raw, o, zero, 90, True, threads=3) < 8e-3
    # the bracketing bf16 neighbour of a large value passes (R13), two steps do not
    up = raw.copy()
    up[3, 5] += 1
    P.check_dx_block(up, o, zero, 90, True, threads=2)
    up[3, 5] += 1
    with pytest.raises(AssertionError):
        P.check_dx_block(up, o, zero, 90, True, threads=2)
    for planted in ((7, 0), (0, 95)):  # a nonzero on a zero row; on a padded column
        bad = raw.copy()
        bad[planted] = 0x3C00
        with pytest.raises(AssertionError):
            P.check_dx_block(bad, o, zero, 90, True, threads=4)
    nan = raw.copy()
    nan[2, 2] = 0x7FC0
    with pytest.raises(AssertionError):
        P.check_dx_block(nan, o, zero, 90, True)
    # fp32: 1e-5 absolute
    raw32 = o.astype(np.float32).view(np.uint32)
    P.check_dx_block(raw32, o, zero, 90, False)
    off = o.astype(np.float32)
    off[10, 10] += np.float32(2e-5)
    with pytest.raises(AssertionError):
        P.check_dx_block(off.view(np.uint32), o, zero, 90, False)


def test_stream_parity_passes_the_oracle_and_catches_planted_misses():
    orc = oracle.get()
    wl = W.small_workload(70, 3001, 3008, num_tiles=5, seed=77)
    inp = W.make_inputs(wl, "cpu")
    xb, tgt, mask, g = W.to_host(inp)
    lo, so, _, _ = orc.fwd(xb, tgt, mask, real_vocab=wl.real_vocab, raise_on_error=False)
    do = orc.bwd(xb, tgt, mask, so, g, real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab)
    logp = torch.from_numpy(lo.astype(np.float32))
    lse = torch.from_numpy(so.astype(np.float32))
    d16 = torch.from_numpy(do).to(torch.bfloat16)
    st = P.stream_parity(orc, inp, logp, lse, d=d16, block=16, tag="oracle as candidate")
    assert st["rows"] == 70 and st["lse_max_abs"] < 1e-6
    bad = d16.clone()
    act = np.flatnonzero(P.effective_active(tgt, mask))
    bad[int(act[-1]), 17] += 0.05  # in the last block
    with pytest.raises(AssertionError):
        P.stream_parity(orc, inp, logp, lse, d=bad, block=16)
    bad_lse = lse.clone()
    bad_lse[69] += 3e-4
    with pytest.raises(AssertionError):
        P.stream_parity(orc, inp, logp, bad_lse, block=32)
    # the extended backward with the oracle's own LSE and entropy
    eo = orc.entropy(xb, real_vocab=wl.real_vocab)
    gen = torch.Generator().manual_seed(3)
    gl, gh = torch.randn(70, generator=gen), torch.randn(70, generator=gen)
    dx = orc.bwd_ex(xb, tgt, mask, so, real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab,
                    ent=eo, g=g, g_lse=gl.double().numpy(), g_ent=gh.double().numpy())
    d32 = torch.from_numpy(dx.astype(np.float32))
    ent = torch.from_numpy(eo.astype(np.float32))
    P.stream_parity(orc, inp, logp, lse, ent=ent, d=d32, g_lse=gl, g_ent=gh, block=25)
    with pytest.raises(AssertionError):  # the plain backward is not the extended one
        P.stream_parity(orc, inp, logp, lse, d=d32, block=25)
