"""The entry point that allocates nothing (rlk_logp_fwd_noalloc), through the C
ABI: its outputs equal rlk_logp_fwd's (with a caller-allocated workspace) bit for
bit, on two calls in a row, the second with a smaller input, so the second call
runs over scratch the first left behind.  Needs an MI355X."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import vocab_selected_token_amd as rlk
import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def bits(t):
    return t.contiguous().view(torch.int32)


def both(inp, shards=1, validate=False):
    wl = inp.wl
    n = wl.num_tokens
    desc = rlk.make_desc(n, wl.real_vocab, wl.padded_vocab, inp.logits.stride(0), wl.num_tiles,
                         shards, validate=validate)
    m = inp.mask.view(torch.uint8)
    ws = rlk.workspace_for(desc, DEV)
    ref = (torch.empty(n, device=DEV), torch.empty(n, device=DEV))
    rlk.rlk_logp_fwd(desc, inp.logits, inp.targets, m, ref[0], ref[1], ws)
    out = (torch.full((n,), 7.0, device=DEV), torch.full((n,), 7.0, device=DEV))
    rlk.rlk_logp_fwd_noalloc(desc, inp.logits, inp.targets, m, out[0], out[1])
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_forward_matches_the_workspace_forward_twice():
    orc = oracle.get()
    cases = [W.small_workload(3000, 151936, 152576, num_tiles=64, sigma=2.5, mask_keep=0.8,
                              ignore_frac=0.05, seed=501),
             W.small_workload(37, 20000, 20008, num_tiles=7, sigma=3.0, mask_keep=0.9,
                              ignore_frac=0.1, seed=502)]
    for i, wl in enumerate(cases):
        print(f"no-alloc call {i}: {wl.num_tokens} x {wl.padded_vocab}, T={wl.num_tiles}",
              flush=True)
        inp = W.make_inputs(wl, DEV)
        ref, out = both(inp, shards=2 if i else 1)
        assert torch.equal(bits(out[0]), bits(ref[0])) and torch.equal(bits(out[1]), bits(ref[1]))
        xb, tgt, mask, _ = W.to_host(inp)
        lo, so, _, _ = orc.fwd(xb, tgt, mask, real_vocab=wl.real_vocab, raise_on_error=False)
        P.check_fwd(out[0].cpu().numpy(), out[1].cpu().numpy(), lo, so,
                    P.effective_active(tgt, mask), f"no-alloc call {i}")


def test_noalloc_forward_validate_and_size_limit():
    wl = W.small_workload(16, 5000, 5008, num_tiles=8, mask_keep=None, ignore_frac=0.0, seed=503)
    inp = W.make_inputs(wl, DEV)
    ref, out = both(inp, validate=True)
    assert torch.equal(bits(out[1]), bits(ref[1]))
    inp.targets[3] = 5003  # a padded column on an active row: an error under VALIDATE
    desc = rlk.make_desc(16, 5000, 5008, inp.logits.stride(0), 8, validate=True)
    logp, lse = torch.empty(16, device=DEV), torch.empty(16, device=DEV)
    with pytest.raises(rlk.RlkError) as ei:
        rlk.rlk_logp_fwd_noalloc(desc, inp.logits, inp.targets, None, logp, lse)
    assert ei.value.status == rlk.RLK_ERR_TARGET_RANGE
    # the status words are cleared by the next validating call
    inp.targets[3] = 7
    rlk.rlk_logp_fwd_noalloc(desc, inp.logits, inp.targets, None, logp, lse)
    big = rlk.make_desc(65537, 151936, 152576, 152576, 64)
    with pytest.raises(rlk.RlkError) as ei:
        rlk.rlk_logp_fwd_noalloc(big, inp.logits, inp.targets, None, logp, lse)
    assert ei.value.status == rlk.RLK_ERR_WORKSPACE
    assert np.isfinite(lse.cpu().numpy()).all()
