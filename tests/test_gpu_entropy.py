"""GPU parity of the extended forward and backward (entropy, LSE and entropy
gradients) and of the differentiable torch interface built on them.

Bars: the forward's logp and LSE bitwise those of rlk_logp_fwd; the entropy
within 1e-4 of the oracle and bitwise identical for every tile grouping; the
per-tile entropy statistic against the oracle's; the extended dlogits within
the dlogits tolerances of the oracle's extended backward, rows that no term
reaches +0 bit for bit; with only grad_logp, bitwise rlk_logp_bwd.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
import vocab_selected_token_amd as rlk
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def fwd_ex(inp, shards=1, validate=False):
    wl = inp.wl
    return rlk.forward_ex(inp.logits, inp.targets, inp.mask, real_vocab=wl.real_vocab,
                          padded_vocab=wl.padded_vocab, num_vocab_tiles=wl.num_tiles,
                          num_virtual_shards=shards, validate=validate)


def bwd_ex(inp, lse, ent, g, gl, gh, dtype):
    wl = inp.wl
    return rlk.backward_ex(inp.logits, inp.targets, inp.mask, lse, ent, g, gl, gh,
                           real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab,
                           out_dtype=dtype, num_vocab_tiles=wl.num_tiles)


def bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def raw_bits(d: torch.Tensor) -> np.ndarray:
    if d.dtype == torch.bfloat16:
        return d.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return d.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def upstream(n, seed):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    return [torch.randn(n, generator=gen).to(DEV) for _ in range(3)]


SMALL = [
    dict(n=37, real=1000, pad=1000, T=7),
    dict(n=64, real=5000, pad=5120, ld=5128, T=64),
    dict(n=16, real=100, pad=128, T=8),
    dict(n=5, real=1, pad=8, T=1),
    dict(n=130, real=151936, pad=152576, T=64),
    dict(n=9, real=3001, pad=3008, T=5, spike=True),
    dict(n=21, real=9000, pad=9000, T=65),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"n{c['n']}_v{c['real']}_p{c['pad']}_T{c['T']}")
def test_small_entropy_and_extended_backward(orc, case):
    print(f"case {case}", flush=True)
    wl = W.small_workload(case["n"], case["real"], case["pad"], ld=case.get("ld"),
                          num_tiles=case["T"], spike_frac=0.3 if case.get("spike") else 0.0,
                          spike=12.0, seed=case["n"] + 2000)
    inp = W.make_inputs(wl, DEV)
    if case["real"] > 8:
        inp.logits[1, 3:8] = float("-inf")  # -inf columns: p = 0, 0 log 0 = 0
    logp, lse, ent = fwd_ex(inp)
    # logp and LSE are bitwise those of the plain forward
    l0, s0 = rlk.forward(inp.logits, inp.targets, inp.mask, real_vocab=wl.real_vocab,
                         padded_vocab=wl.padded_vocab, num_vocab_tiles=wl.num_tiles)
    assert torch.equal(bits(logp), bits(l0)) and torch.equal(bits(lse), bits(s0))
    for s in sorted({2, 3, 8, case["T"]} & set(range(2, case["T"] + 1))):
        _, _, e2 = fwd_ex(inp, shards=s)
        assert torch.equal(bits(e2), bits(ent)), f"S={s} entropy"
    xb, tgt, mask, g = W.to_host(inp)
    lo, so, _, _ = orc.fwd(xb, tgt, mask, real_vocab=wl.real_vocab, raise_on_error=False)
    eo = orc.entropy(xb, real_vocab=wl.real_vocab)
    P.check_fwd(logp.cpu().numpy(), lse.cpu().numpy(), lo, so,
                P.effective_active(tgt, mask), str(case))
    P.check_entropy(ent.cpu().numpy(), eo, str(case))
    act = P.effective_active(tgt, mask)
    g1, gl, gh = upstream(wl.num_tokens, case["n"])
    # the oracle's backward takes the oracle's own LSE and entropy, never the GPU's
    lse_h, ent_h = so, eo
    combos = [(g1, None, None), (None, gl, None), (None, None, gh), (g1, gl, gh)]
    for dt in (torch.float32, torch.bfloat16):
        for gg, ggl, ggh in combos:
            d = bwd_ex(inp, lse, ent, gg, ggl, ggh, dt)
            do = orc.bwd_ex(xb, tgt, mask, lse_h, real_vocab=wl.real_vocab,
                            padded_vocab=wl.padded_vocab, ent=ent_h,
                            g=None if gg is None else gg.double().cpu().numpy(),
                            g_lse=None if ggl is None else ggl.double().cpu().numpy(),
                            g_ent=None if ggh is None else ggh.double().cpu().numpy(),
                            raise_on_error=False)
            zero = ~act if (ggl is None and ggh is None) else np.zeros_like(act)
            P.check_bwd_ex(P.dlogits_host(d), do, zero, wl.real_vocab, dt == torch.bfloat16,
                           f"{case} {dt} g={gg is not None} gl={ggl is not None} "
                           f"gh={ggh is not None}", raw_bits(d))
        # only grad_logp: bitwise the plain backward
        d_ex = bwd_ex(inp, lse, ent, g1, None, None, dt)
        d_pl = rlk.backward(inp.logits, inp.targets, inp.mask, lse, g1, real_vocab=wl.real_vocab,
                            padded_vocab=wl.padded_vocab, out_dtype=dt,
                            num_vocab_tiles=wl.num_tiles)
        assert torch.equal(bits(d_ex), bits(d_pl))


@pytest.mark.parametrize("shape", [(40, 151936, 151936, 64), (24, 3001, 3008, 5),
                                   (16, 100, 128, 8)])
def test_stage1_entropy_statistic(orc, shape):
    n, real, pad, t = shape
    wl = W.small_workload(n, real, pad, num_tiles=t, seed=6)
    inp = W.make_inputs(wl, DEV)
    inp.logits[1, :real] = float("-inf")
    inp.logits[2, :real // 2] = float("-inf")
    desc = rlk.make_desc(n, real, pad, inp.logits.stride(0), t)
    ws = torch.empty(rlk.rlk_logp_ex_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    logp, lse, ent = (torch.empty(n, device=DEV) for _ in range(3))
    rlk.rlk_logp_fwd_ex(desc, inp.logits, inp.targets, None, logp, lse, ent, ws)
    torch.cuda.synchronize()
    part = (n * t * 4 + 255) // 256 * 256
    base = 256 + 2 * part
    pe = ws[base:base + n * t * 4].view(torch.float32).view(n, t).double().cpu().numpy()
    ps = ws[256 + part:256 + part + n * t * 4].view(torch.float32).view(n, t).double().cpu().numpy()
    xb, _, _, _ = W.to_host(inp)
    _, os_, oe = orc.tile_partials(xb, real_vocab=real, padded_vocab=pad, num_tiles=t,
                                   with_entropy=True)
    assert (pe[os_ == 0] == 0).all()  # identity tiles carry 0
    err = np.abs(pe - oe)
    assert (err <= 1e-5 * (np.abs(oe) + os_) + 1e-30).all(), err.max()


def test_entropy_closed_forms():
    v = 151936
    n = 6
    wl = W.small_workload(n, v, mask_keep=None, ignore_frac=0.0, seed=3)
    inp = W.make_inputs(wl, DEV)
    inp.logits[0, :] = 0.0
    inp.logits[1, :] = -7.25
    inp.logits[2, :] = float("-inf")
    inp.logits[2, 1234] = 5.0
    inp.logits[3, :] = float("-inf")
    inp.logits[3, [7, 80000, v - 1]] = 2.5
    inp.logits[4, :] = float("-inf")
    inp.targets[2] = 1234
    inp.targets[3] = 7
    m = torch.ones(n, dtype=torch.bool, device=DEV)
    m[4] = False
    logp, lse, ent = rlk.forward_ex(inp.logits, inp.targets, m, real_vocab=v)
    e = ent.double().cpu().numpy()
    assert abs(e[0] - math.log(v)) <= 1e-4 and abs(e[1] - math.log(v)) <= 1e-4
    assert e[2] == 0.0
    assert abs(e[3] - math.log(3.0)) <= 1e-6
    assert math.isnan(e[4])


def test_autograd_interface(orc):
    """A loss on all three outputs through torch autograd: logits.grad equals the
    oracle's extended backward with the loss's upstream gradients."""
    wl = W.small_workload(48, 20000, 20008, seed=12)
    inp = W.make_inputs(wl, DEV)
    x = inp.logits.clone().requires_grad_(True)
    logp, lse, ent = rlk.selected_token_logprob(x, inp.targets, inp.mask,
                                                real_vocab=wl.real_vocab,
                                                num_vocab_tiles=wl.num_tiles)
    w1, w2, w3 = upstream(wl.num_tokens, 99)
    loss = (w1 * logp).sum() + (w2 * lse).sum() + (w3 * ent).sum()
    loss.backward()
    assert x.grad.dtype == torch.bfloat16 and x.grad.shape == x.shape
    xb, tgt, mask, _ = W.to_host(inp)
    _, so, _, _ = orc.fwd(xb, tgt, mask, real_vocab=wl.real_vocab)
    eo = orc.entropy(xb, real_vocab=wl.real_vocab)
    do = orc.bwd_ex(xb, tgt, mask, so, real_vocab=wl.real_vocab,
                    padded_vocab=wl.padded_vocab, ent=eo,
                    g=w1.double().cpu().numpy(), g_lse=w2.double().cpu().numpy(),
                    g_ent=w3.double().cpu().numpy())
    P.check_bwd_ex(P.dlogits_host(x.grad[:, :wl.padded_vocab]), do,
                   np.zeros(wl.num_tokens, dtype=bool), wl.real_vocab, True, "autograd",
                   raw_bits(x.grad[:, :wl.padded_vocab]))
    assert (bits(x.grad[:, wl.padded_vocab:]) == 0).all()


def test_policy_gradient_consumer(orc):
    """A loss of the kind the pages' RL runs train with: an advantage-weighted logp
    term plus a KL penalty of coefficient 0.01 against reference log-probabilities
    (k3 estimator exp(r - logp) - (r - logp) - 1), over active tokens.  The
    gradient through the op equals the oracle backward with g = dloss/dlogp."""
    wl = W.small_workload(64, 151936, 152576, seed=13)
    inp = W.make_inputs(wl, DEV)
    x = inp.logits.clone().requires_grad_(True)
    logp, _, _ = rlk.selected_token_logprob(x, inp.targets, inp.mask, real_vocab=wl.real_vocab)
    gen = torch.Generator(device="cpu").manual_seed(5)
    adv = torch.randn(wl.num_tokens, generator=gen).to(DEV)
    ref = (logp.detach() + 0.1 * torch.randn(wl.num_tokens, generator=gen).to(DEV))
    act = (inp.mask & (inp.targets != -100)).float()
    diff = ref - logp
    k3 = torch.exp(diff) - diff - 1.0
    loss = ((-adv * logp + 0.01 * k3) * act).sum() / act.sum()
    loss.backward()
    # dloss/dlogp by hand, in float64 from the same fp32 logp
    lp = logp.detach().double().cpu().numpy()
    a = act.double().cpu().numpy()
    g = (-adv.double().cpu().numpy() + 0.01 * (1.0 - np.exp(ref.double().cpu().numpy() - lp)))
    g = g * a / a.sum()
    xb, tgt, mask, _ = W.to_host(inp)
    _, so, _, _ = orc.fwd(xb, tgt, mask, real_vocab=wl.real_vocab)
    do = orc.bwd(xb, tgt, mask, so, g, real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab)
    P.check_bwd(P.dlogits_host(x.grad), do, P.effective_active(tgt, mask), wl.real_vocab, True,
                "policy gradient", raw_bits(x.grad))


def test_microbatch_1024_entropy_and_extended_backward(orc):
    inp = W.make_inputs(W.MICROBATCH_1024, DEV)
    wl = inp.wl
    logp, lse, ent = fwd_ex(inp)
    g1, gl, gh = upstream(wl.num_tokens, 3)
    d = bwd_ex(inp, lse, ent, g1, gl, gh, torch.float32)
    inp.grad = g1
    stats = P.stream_parity(orc, inp, logp, lse, ent=ent, d=d, g_lse=gl, g_ent=gh, block=256,
                            tag="mb1024 extended")
    print(stats, flush=True)


def test_large_32k_entropy_full(orc):
    """The 32768-row workload through the extended forward and backward: entropy
    bitwise the same at S = 8, and every row's logp, LSE, entropy and bf16 dX (with
    the LSE and entropy gradients) against the oracle's own values."""
    wl = W.LARGE_32K
    inp = W.make_inputs(wl, DEV)
    logp, lse, ent = fwd_ex(inp)
    _, _, e8 = fwd_ex(inp, shards=8)
    assert torch.equal(bits(e8), bits(ent))
    del e8
    g1, gl, gh = upstream(wl.num_tokens, 4)
    d = bwd_ex(inp, lse, ent, g1, gl, gh, torch.bfloat16)
    inp.grad = g1
    stats = P.stream_parity(orc, inp, logp, lse, ent=ent, d=d, g_lse=gl, g_ent=gh, block=1024,
                            tag="32k extended")
    print(stats, flush=True)


def test_extended_validate_and_bad_targets():
    wl = W.small_workload(12, 5000, 5008, mask_keep=None, ignore_frac=0.0, seed=19)
    inp = W.make_inputs(wl, DEV)
    logp0, lse0, ent0 = fwd_ex(inp, validate=True)
    g1, gl, gh = upstream(wl.num_tokens, 21)
    d0 = bwd_ex(inp, lse0, ent0, g1, gl, gh, torch.float32)
    inp.targets[4] = 5003  # a padded column: an error on an effective-active row
    with pytest.raises(rlk.RlkError) as ei:
        fwd_ex(inp, validate=True)
    assert ei.value.status == rlk.RLK_ERR_TARGET_RANGE
    logp, lse, ent = fwd_ex(inp)
    keep = torch.arange(12, device=DEV) != 4
    assert torch.isnan(logp[4]) and torch.equal(bits(lse), bits(lse0))
    assert torch.equal(bits(ent), bits(ent0)) and torch.equal(bits(logp[keep]), bits(logp0[keep]))
    with pytest.raises(rlk.RlkError) as ei:
        rlk.backward_ex(inp.logits, inp.targets, inp.mask, lse, ent, g1, gl, gh,
                        real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab,
                        num_vocab_tiles=wl.num_tiles, validate=True)
    assert ei.value.status == rlk.RLK_ERR_TARGET_RANGE
    d = bwd_ex(inp, lse, ent, g1, gl, gh, torch.float32)
    assert torch.isnan(d[4, :5000]).all() and (bits(d[4, 5000:]) == 0).all()
    assert torch.equal(bits(d[keep]), bits(d0[keep]))
    # an inactive row with a bad target is not an error: only its LSE/entropy terms remain
    m = torch.ones(12, dtype=torch.bool, device=DEV)
    m[4] = False
    logp, lse, ent = rlk.forward_ex(inp.logits, inp.targets, m, real_vocab=wl.real_vocab,
                                    padded_vocab=wl.padded_vocab, num_vocab_tiles=wl.num_tiles,
                                    validate=True)
    d = rlk.backward_ex(inp.logits, inp.targets, m, lse, ent, g1, gl, gh,
                        real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab,
                        num_vocab_tiles=wl.num_tiles, validate=True)
    assert not torch.isnan(d[4]).any() and (d[4, :5000] != 0).any()


def test_extended_side_stream():
    wl = W.small_workload(40, 20000, 20000, seed=23)
    inp = W.make_inputs(wl, DEV)
    ref = fwd_ex(inp)
    g1, gl, gh = upstream(wl.num_tokens, 22)
    dref = bwd_ex(inp, ref[1], ref[2], g1, gl, gh, torch.bfloat16)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = rlk.forward_ex(inp.logits, inp.targets, inp.mask, real_vocab=wl.real_vocab,
                             num_vocab_tiles=wl.num_tiles, stream=s)
        d = rlk.backward_ex(inp.logits, inp.targets, inp.mask, out[1], out[2], g1, gl, gh,
                            real_vocab=wl.real_vocab, out_dtype=torch.bfloat16,
                            num_vocab_tiles=wl.num_tiles, stream=s)
    s.synchronize()
    for a, b in zip(out, ref):
        assert torch.equal(bits(a), bits(b))
    assert torch.equal(bits(d), bits(dref))
