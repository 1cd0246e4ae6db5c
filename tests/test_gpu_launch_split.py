"""A batch split into many launches gives the same bits as one launch.

A dispatch holds its grid size in 32 bits of threads: at 2^32 threads the launch
fails, and above it the size wraps around and the kernel runs on a fraction of
its grid with no error.  Every launcher therefore splits its work into launches
of at most 2^31 threads, each told where its part of the batch starts.  The
backward of the 32K-row bench workload is one launch of 315M threads; a batch of
about 447K rows of 152576 columns (136 GB of bf16 logits, which fits in this
GPU's memory next to its bf16 dlogits) needs more than 2^32.  The RLK_MAX_LAUNCH_THREADS
environment variable (read once per process) lowers the limit so that small
shapes run in hundreds of launches; what a row, tile or block computes does not
depend on the split, so every output must match the single-launch run bit for
bit.  Needs an MI355X.
"""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

import pytest
import torch

import vocab_selected_token_amd as rlk
import workloads as W
from tests.split_child import make_case, run_all

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")
ROOT = Path(__file__).resolve().parent.parent


def test_split_launches_give_the_same_bits(tmp_path):
    """The library reads the limit once per process, so each lowered limit runs in
    a child process (tests/split_child.py) on the same seeded case; its output bits
    must equal this process's, which runs every kernel as one launch."""
    ref = run_all(*make_case())
    for limit in (1024, 5000, 65536):
        print(f"launch limit {limit} threads (child process)", flush=True)
        out = tmp_path / f"bits_{limit}.pt"
        env = dict(os.environ, RLK_MAX_LAUNCH_THREADS=str(limit))
        r = subprocess.run([sys.executable, "-u", "-m", "tests.split_child", str(out)], cwd=ROOT,
                           env=env, capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, f"child with limit {limit} failed:\n{r.stdout[-2000:]}\n{r.stderr[-3000:]}"
        got = torch.load(out, weights_only=True)
        assert set(got) == set(ref)
        for a, b in zip(ref["lmhead"], got["lmhead_s3"]):
            assert torch.equal(a, b), "three virtual shards differ from one"
        for key in ref:
            for a, b in zip(ref[key], got[key]):
                assert torch.equal(a, b), f"{key} differs with a {limit}-thread launch limit"


def test_unit_schedule_fallback_gives_the_same_bits(tmp_path):
    """The one-launch unit schedule bounds each block's wait for the other units
    of its row; past the bound the block computes the row's partials itself.
    RLK_FB_SPIN_LIMIT=0 (read once per process) sends every block down that path
    at once: a child process runs the same case and its bits must equal this
    process's, which waits for the published partials."""
    ref = run_all(*make_case())
    out = tmp_path / "bits_fallback.pt"
    env = dict(os.environ, RLK_FB_SPIN_LIMIT="0")
    print("spin limit 0 (child process)", flush=True)
    r = subprocess.run([sys.executable, "-u", "-m", "tests.split_child", str(out)], cwd=ROOT,
                       env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"child failed:\n{r.stdout[-2000:]}\n{r.stderr[-3000:]}"
    got = torch.load(out, weights_only=True)
    # status word 2 counts the blocks that computed their row's partials themselves:
    # none here, all 300 rows x 8 units in the child
    for key in ("one_fallbacks", "one_ex_fallbacks"):
        assert ref[key][0].item() == 0, key
        assert got[key][0].item() == 300 * 8, key
    for key in ref:
        if key.endswith("_fallbacks"):
            continue
        for a, b in zip(ref[key], got[key]):
            assert torch.equal(a, b), f"{key} differs when every block computes its row itself"


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
