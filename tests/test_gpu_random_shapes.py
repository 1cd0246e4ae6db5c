"""Seeded sweep of ragged shapes through every materialised-logits entry point.

For each drawn shape (tokens, real and padded vocabulary, row stride, tile and
shard counts, mask and ignore rates, logit scale, a few -inf columns):
  * rlk_logp_fwd / rlk_logp_bwd (fp32 and bf16) against the oracle;
  * every drawn shard count gives the bits of S = 1;
  * rlk_logp_fwd_bwd gives the bits of the separate calls;
  * rlk_logp_fwd_ex gives the same logp and LSE bits, and its entropy matches
    the oracle; rlk_logp_bwd_ex matches the oracle's extended backward;
  * rlk_logp_fwd_bwd_ex gives the bits of rlk_logp_fwd_ex then rlk_logp_bwd_ex.
The shapes are drawn once from a fixed seed, so the sweep is reproducible.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
import vocab_selected_token_amd as rlk
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def draw_cases(count: int, seed: int):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        real = int(rng.choice([1, 7, 64, 255, 1000, 2374 * 2 + 5, 9999, 40000]))
        pad = real + int(rng.choice([0, 0, 3, 8, 129, 640]))
        t_max = min(pad, 1024)
        T = int(rng.choice([t for t in (1, 2, 3, 7, 16, 63, 64, 65, 200, 1024) if t <= t_max]))
        ld = (pad + 7) // 8 * 8 + int(rng.choice([0, 0, 8, 64]))
        n = int(rng.choice([1, 2, 17, 64, 100, 257]))
        S = int(rng.choice([s for s in (1, 2, 3, 4, 8, 64) if s <= T]))
        cases.append(dict(i=i, n=n, real=real, pad=pad, ld=ld, T=T, S=S,
                          sigma=float(rng.choice([0.5, 2.0, 6.0])),
                          mask_keep=float(rng.choice([0.5, 0.9, 1.1])),
                          ignore=float(rng.choice([0.0, 0.1])), seed=int(rng.integers(1 << 30))))
    return cases


# RLK_RANDOM_SHAPES=300 runs the longer stress sweep the design notes quote
CASES = draw_cases(int(os.environ.get("RLK_RANDOM_SHAPES", "24")), seed=20261202)


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"{c['i']}_n{c['n']}_v{c['real']}_p{c['pad']}"
                                                  f"_ld{c['ld']}_T{c['T']}_S{c['S']}")
def test_random_shape(orc, c):
    print(f"case {c}", flush=True)
    wl = W.small_workload(c["n"], c["real"], c["pad"], ld=c["ld"], num_tiles=c["T"],
                          sigma=c["sigma"], mask_keep=c["mask_keep"] if c["mask_keep"] <= 1 else None,
                          ignore_frac=c["ignore"], seed=c["seed"])
    inp = W.make_inputs(wl, DEV)
    if c["real"] > 10:
        inp.logits[0, 2:5] = float("-inf")
    kw = dict(real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab, num_vocab_tiles=wl.num_tiles)
    logp, lse = rlk.forward(inp.logits, inp.targets, inp.mask, **kw)
    xb, tgt, mask, g = W.to_host(inp)
    act = P.effective_active(tgt, mask)
    lo, so, _, _ = orc.fwd(xb, tgt, mask, real_vocab=wl.real_vocab, raise_on_error=False)
    P.check_fwd(logp.cpu().numpy(), lse.cpu().numpy(), lo, so, act, str(c))
    ls, ss = rlk.forward(inp.logits, inp.targets, inp.mask, num_virtual_shards=c["S"], **kw)
    assert torch.equal(bits(ls), bits(logp)) and torch.equal(bits(ss), bits(lse))
    do = orc.bwd(xb, tgt, mask, so, g, real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab,
                 raise_on_error=False)
    for dt in (torch.float32, torch.bfloat16):
        d = rlk.backward(inp.logits, inp.targets, inp.mask, lse, inp.grad, out_dtype=dt, **kw)
        raw = bits(d).cpu().numpy().view(np.uint16 if dt == torch.bfloat16 else np.uint32)
        P.check_bwd(P.dlogits_host(d), do, act, wl.real_vocab, dt == torch.bfloat16, str(c), raw)
        if c["T"] <= 1024:
            l1, s1, d1 = rlk.forward_backward(inp.logits, inp.targets, inp.mask, inp.grad,
                                              out_dtype=dt, num_virtual_shards=c["S"], **kw)
            assert torch.equal(bits(l1), bits(logp)) and torch.equal(bits(s1), bits(lse))
            assert torch.equal(bits(d1), bits(d))
    le, se, ent = rlk.forward_ex(inp.logits, inp.targets, inp.mask, num_virtual_shards=c["S"],
                                 **kw)
    assert torch.equal(bits(le), bits(logp)) and torch.equal(bits(se), bits(lse))
    P.check_entropy(ent.cpu().numpy(), orc.entropy(xb, real_vocab=wl.real_vocab), str(c))
    gen = torch.Generator(device="cpu").manual_seed(c["seed"])
    gl, gh = (torch.randn(wl.num_tokens, generator=gen).to(DEV) for _ in range(2))
    dx = rlk.backward_ex(inp.logits, inp.targets, inp.mask, lse, ent, inp.grad, gl, gh, **kw)
    # the oracle's side takes the oracle's own LSE and entropy
    dox = orc.bwd_ex(xb, tgt, mask, so, real_vocab=wl.real_vocab,
                     padded_vocab=wl.padded_vocab, ent=orc.entropy(xb, real_vocab=wl.real_vocab),
                     g=g,
                     g_lse=gl.double().cpu().numpy(), g_ent=gh.double().cpu().numpy(),
                     raise_on_error=False)
    P.check_bwd_ex(P.dlogits_host(dx), dox, np.zeros(wl.num_tokens, dtype=bool), wl.real_vocab,
                   False, str(c), bits(dx).cpu().numpy().view(np.uint32))
    # the extended forward and backward in one launch: the bits of the two calls
    l4, s4, e4, d4 = rlk.forward_backward_ex(inp.logits, inp.targets, inp.mask, inp.grad, gl, gh,
                                             num_virtual_shards=c["S"], **kw)
    for a, b, name in ((l4, le, "logp"), (s4, se, "lse"), (e4, ent, "entropy"), (d4, dx, "dX")):
        na = torch.isnan(a)
        assert torch.equal(na, torch.isnan(b)), f"one launch extended {name}: NaN pattern"
        zero = torch.zeros((), dtype=bits(a).dtype, device=DEV)
        assert torch.equal(torch.where(na, zero, bits(a)), torch.where(na, zero, bits(b))), \
            f"one launch extended {name}: bits differ"
