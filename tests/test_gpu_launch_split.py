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


def test_backward_split_at_full_size():
    """The split without the override: 224,000 rows of 152576 columns (68 GB of bf16
    logits, and as much bf16 dX) put the backward at 224,000 x 75 blocks of 128
    threads, past 2^31 threads, so it runs as two launches, the second starting
    inside row 223,696.  Rows on both sides of that point, and others, match the
    oracle and match the same rows computed in a small batch bit for bit; every
    inactive row and every padded column is +0."""
    import numpy as np

    import oracle
    from tests import parity as P

    n, v_real, v_pad = 224_000, 151_936, 152_576
    need = 2 * n * v_pad * 2 + (4 << 30)
    torch.cuda.empty_cache()  # blocks cached by earlier tests in this process
    free, _ = torch.cuda.mem_get_info()
    assert free >= need, f"needs {need / 2**30:.0f} GiB of free device memory, {free / 2**30:.0f} free"
    assert n * 75 * 128 > 2**31 > 223_696 * 75 * 128  # two launches; the cut is in row 223,696
    wl = W.small_workload(n, v_real, v_pad, num_tiles=64, sigma=2.5, mask_keep=0.85,
                          ignore_frac=0.05, seed=2024, dlogits_dtype="bf16")
    print("generating 224000 x 152576 bf16 logits", flush=True)
    inp = W.make_inputs(wl, DEV)
    kw = dict(real_vocab=v_real, padded_vocab=v_pad, num_vocab_tiles=64)
    logp, lse = rlk.forward(inp.logits, inp.targets, inp.mask, **kw)
    d = rlk.backward(inp.logits, inp.targets, inp.mask, lse, inp.grad, out_dtype=torch.bfloat16,
                     **kw)
    torch.cuda.synchronize()
    print("forward and backward done", flush=True)
    tgt = inp.targets.cpu().numpy()
    mask = inp.mask.cpu().numpy()
    act = P.effective_active(tgt, mask)
    act_t = torch.from_numpy(act).to(DEV)
    dbits = d.view(torch.int16)
    for r0 in range(0, n, 8192):
        sl = slice(r0, min(n, r0 + 8192))
        assert not bool((dbits[sl][~act_t[sl]] != 0).any()), f"inactive rows near {r0}"
        assert not bool((dbits[sl, v_real:] != 0).any()), f"padded columns near {r0}"
    rng = np.random.default_rng(5)
    rows = np.array(sorted({0, 1, 223_695, 223_696, 223_697, n - 1} |
                           set(rng.choice(n, 10, replace=False).tolist())))
    rows_t = torch.from_numpy(rows).to(DEV)
    # the same rows in a batch of their own: one launch per kernel
    sub = [t[rows_t].contiguous() for t in (inp.logits, inp.targets, inp.mask, inp.grad)]
    lp_s, lse_s = rlk.forward(sub[0], sub[1], sub[2], **kw)
    d_s = rlk.backward(sub[0], sub[1], sub[2], lse_s, sub[3], out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    assert torch.equal(lp_s.view(torch.int32), logp[rows_t].view(torch.int32))
    assert torch.equal(lse_s.view(torch.int32), lse[rows_t].view(torch.int32))
    assert torch.equal(d_s.view(torch.int16), dbits[rows_t])
    orc = oracle.get()
    bits, t_s, m_s, g_s = W.to_host(inp, rows)
    lo, so, _, _ = orc.fwd(bits, t_s, m_s, real_vocab=v_real, raise_on_error=False)
    P.check_fwd(logp[rows_t].cpu().numpy(), lse[rows_t].cpu().numpy(), lo, so, act[rows],
                "224k")
    do = orc.bwd(bits, t_s, m_s, so, g_s, real_vocab=v_real, padded_vocab=v_pad)
    sel = d[rows_t]
    P.check_bwd(P.dlogits_host(sel), do, act[rows], v_real, True, "224k bwd",
                sel.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    del inp, d, dbits, sub
    torch.cuda.empty_cache()
