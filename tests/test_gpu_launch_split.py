"""A batch split into many launches gives the same bits as one launch.

A dispatch holds its grid size in 32 bits of threads: at 2^32 threads the launch
fails, and above it the size wraps around and the kernel runs on a fraction of
its grid with no error.  Every launcher therefore splits its work into launches
of at most 2^31 threads, each told where its part of the batch starts.  The
backward of the 32K-row bench workload is one launch of 315M threads; a batch of
about 447K rows of 152576 columns (136 GB of bf16 logits, which fits in this
GPU's memory next to its bf16 dlogits) needs more than 2^32.  The RLK_MAX_LAUNCH_THREADS
environment variable lowers the limit so that small shapes run in hundreds of
launches; what a row, tile or block computes does not depend on the split, so
every output must match the single-launch run bit for bit.  Needs an MI355X.
"""
from __future__ import annotations

import pytest
import torch

import vocab_selected_token_amd as rlk
import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def run_all(inp, wl, lm):
    kw = dict(real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab, num_vocab_tiles=wl.num_tiles)
    out = {}
    out["fwd"] = rlk.forward(inp.logits, inp.targets, inp.mask, **kw)
    out["fwd_s4"] = rlk.forward(inp.logits, inp.targets, inp.mask, num_virtual_shards=4, **kw)
    logp, lse, ent = rlk.forward_ex(inp.logits, inp.targets, inp.mask, **kw)
    out["fwd_ex"] = (logp, lse, ent)
    # 16 tiles per shard: stage 1 takes its one-wave-block form
    out["fwd_ex_s4"] = rlk.forward_ex(inp.logits, inp.targets, inp.mask, num_virtual_shards=4,
                                      **kw)
    for dt in (torch.float32, torch.bfloat16):
        out[f"bwd_{dt}"] = (rlk.backward(inp.logits, inp.targets, inp.mask, lse, inp.grad,
                                         out_dtype=dt, **kw),)
        out[f"one_{dt}"] = rlk.forward_backward(inp.logits, inp.targets, inp.mask, inp.grad,
                                                out_dtype=dt, **kw)
    gl = torch.linspace(-1.0, 1.0, wl.num_tokens, device=DEV)
    out["bwd_ex"] = (rlk.backward_ex(inp.logits, inp.targets, inp.mask, lse, ent, inp.grad, gl,
                                     -gl, **kw),)
    h, w, tg, v_real, v_pad, t = lm
    out["lmhead"] = rlk.fused_lmhead(h, w, tg, real_vocab=v_real, padded_vocab=v_pad,
                                     num_vocab_tiles=t)
    out["lmhead_s3"] = rlk.fused_lmhead(h, w, tg, real_vocab=v_real, padded_vocab=v_pad,
                                        num_vocab_tiles=t, num_virtual_shards=3)
    torch.cuda.synchronize()
    return {k: tuple(bits(x).cpu() for x in v) for k, v in out.items()}


@pytest.fixture(scope="module")
def case():
    wl = W.small_workload(300, 5000, 5120, num_tiles=64, sigma=2.0, mask_keep=0.8,
                          ignore_frac=0.05, seed=77)
    inp = W.make_inputs(wl, DEV)
    gen = torch.Generator(device="cpu").manual_seed(78)
    n_tok, k, v_real, v_pad, t = 300, 128, 5000, 5120, 16
    h = (torch.randn(n_tok, k, generator=gen)).to(torch.bfloat16).to(DEV)
    w = (torch.randn(v_pad, k, generator=gen) * 0.1).to(torch.bfloat16).to(DEV)
    tg = torch.randint(0, v_real, (n_tok,), generator=gen, dtype=torch.int32).to(DEV)
    lm = (h, w, tg, v_real, v_pad, t)
    return inp, wl, lm, run_all(inp, wl, lm)


@pytest.mark.parametrize("limit", [1024, 5000, 65536])
def test_split_launches_give_the_same_bits(case, limit, monkeypatch):
    inp, wl, lm, ref = case
    print(f"launch limit {limit} threads", flush=True)
    monkeypatch.setenv("RLK_MAX_LAUNCH_THREADS", str(limit))
    got = run_all(inp, wl, lm)
    for a, b in zip(ref["lmhead"], got["lmhead_s3"]):
        assert torch.equal(a, b), "three virtual shards differ from one"
    for key in ref:
        for a, b in zip(ref[key], got[key]):
            assert torch.equal(a, b), f"{key} differs with a {limit}-thread launch limit"
