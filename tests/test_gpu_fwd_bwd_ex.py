"""GPU parity of the extended forward and backward in one launch
(rlk_logp_fwd_bwd_ex).

Bars, all through the C ABI:
  * bit for bit against rlk_logp_fwd_ex followed by rlk_logp_bwd_ex on the same
    inputs (logp, LSE, entropy and dlogits; NaN where they are NaN), with every
    combination of the three upstream gradients, fp32 and bf16 dX, on geometries
    that take the unit schedule and on ones that run the two calls;
  * against the CPU oracle on every row of two workloads, the oracle's backward
    fed its own LSE and entropy;
  * no block falls back to computing its row alone (status word 2 stays 0).
Inputs come from workloads.py (seeded, synthetic).
"""
from __future__ import annotations

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


def bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def assert_same(a4, b4, what):
    """Bit for bit, NaN where NaN (any payload).  No boolean indexing: a 32K-row dX
    has more elements than a mask-select handles."""
    for a, b, name in zip(a4, b4, ("logp", "lse", "entropy", "dlogits")):
        na, nb = torch.isnan(a), torch.isnan(b)
        assert torch.equal(na, nb), f"{what} {name}: NaN pattern differs"
        if bool(na.any()):
            zero = torch.zeros((), dtype=bits(a).dtype, device=a.device)
            same = torch.equal(torch.where(na, zero, bits(a)), torch.where(nb, zero, bits(b)))
        else:
            same = torch.equal(bits(a), bits(b))
        assert same, f"{what} {name}: bits differ"


def upstream(n, seed):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    return [torch.randn(n, generator=gen).to(DEV) for _ in range(3)]


def one(inp, g, gl, gh, dtype, workspace=None, validate=False, mask="wl"):
    wl = inp.wl
    return rlk.forward_backward_ex(inp.logits, inp.targets, inp.mask if mask == "wl" else mask,
                                   g, gl, gh, real_vocab=wl.real_vocab,
                                   padded_vocab=wl.padded_vocab, num_vocab_tiles=wl.num_tiles,
                                   out_dtype=dtype, workspace=workspace, validate=validate)


def two(inp, g, gl, gh, dtype):
    wl = inp.wl
    logp, lse, ent = rlk.forward_ex(inp.logits, inp.targets, inp.mask, real_vocab=wl.real_vocab,
                                    padded_vocab=wl.padded_vocab, num_vocab_tiles=wl.num_tiles)
    d = rlk.backward_ex(inp.logits, inp.targets, inp.mask, lse, ent, g, gl, gh,
                        real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab, out_dtype=dtype,
                        num_vocab_tiles=wl.num_tiles)
    return logp, lse, ent, d


def desc_of(wl):
    return rlk.make_desc(wl.num_tokens, wl.real_vocab, wl.padded_vocab, wl.ld_logits,
                         wl.num_tiles)


# unit-schedule geometries (tiles of four passes, bounds off the 8-column grid, a
# short last unit, 8-column tiles, whole padding tiles) and ones that run the two
# calls (T above 64, tiles wider than four passes)
SHAPES = [
    dict(n=300, real=151936, pad=152576, T=64, units=True),
    dict(n=64, real=5000, pad=5120, ld=5128, T=64, units=True),
    dict(n=9, real=3001, pad=3008, T=5, spike=True, units=True),
    dict(n=40, real=515, pad=600, T=64, units=True),
    dict(n=20, real=700, pad=2048, T=64, units=True),
    dict(n=21, real=9000, pad=9000, T=65, units=False),
    dict(n=12, real=4000, pad=4096, T=1, units=False),
]
COMBOS = [(True, False, False), (False, True, False), (False, False, True), (True, True, True)]


@pytest.mark.parametrize("case", SHAPES,
                         ids=lambda c: f"n{c['n']}_v{c['real']}_p{c['pad']}_T{c['T']}")
def test_bitwise_equal_to_the_two_extended_calls(case):
    print(f"case {case}", flush=True)
    wl = W.small_workload(case["n"], case["real"], case["pad"], ld=case.get("ld"),
                          num_tiles=case["T"], spike_frac=0.3 if case.get("spike") else 0.0,
                          spike=12.0, seed=case["n"] + 7000)
    d = desc_of(wl)
    n = wl.num_tokens
    # the geometry takes the unit schedule exactly when rlk_logp_fwd_bwd asks for slots
    assert (rlk.rlk_logp_fwd_bwd_workspace_bytes(d) > 256) == case["units"]
    assert rlk.rlk_logp_fwd_bwd_ex_workspace_bytes(d) >= (
        max(256 + 16 * n * wl.num_tiles, rlk.rlk_logp_ex_workspace_bytes(d)) if case["units"]
        else rlk.rlk_logp_ex_workspace_bytes(d))
    inp = W.make_inputs(wl, DEV)
    if n > 6:
        inp.logits[1, :wl.real_vocab] = float("-inf")  # no finite logit
        inp.logits[2, wl.real_vocab - 1] = float("nan")
        inp.logits[3, 0] = float("inf")
        inp.mask[1] = True
        inp.targets[4] = wl.real_vocab + 3  # a bad target on an active row
        inp.mask[4] = True
        inp.mask[5] = False  # inactive: reached by the LSE and entropy terms only
        inp.logits[5].view(torch.int16)[wl.real_vocab // 2] = -1  # all-payload NaN
    g, gl, gh = upstream(n, case["n"])
    ws = torch.empty(rlk.rlk_logp_fwd_bwd_ex_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    for dt in (torch.float32, torch.bfloat16):
        for use in COMBOS:
            args = [t if u else None for t, u in zip((g, gl, gh), use)]
            out = one(inp, *args, dt, workspace=ws)
            torch.cuda.synchronize()
            if case["units"]:
                assert ws[:12].view(torch.int32)[2].item() == 0, f"{case} {dt} {use}: fell back"
            assert_same(out, two(inp, *args, dt), f"{case} {dt} {use}")


def test_two_call_path_with_a_smaller_workspace():
    """Where the unit schedule fits but the workspace holds only the two calls'
    partials, the two calls run: the same bits."""
    wl = W.small_workload(48, 151936, 152576, num_tiles=64, seed=77)
    inp = W.make_inputs(wl, DEV)
    g, gl, gh = upstream(wl.num_tokens, 5)
    small = torch.empty(rlk.rlk_logp_ex_workspace_bytes(desc_of(wl)), dtype=torch.uint8,
                        device=DEV)
    assert small.numel() < rlk.rlk_logp_fwd_bwd_ex_workspace_bytes(desc_of(wl))
    for dt in (torch.float32, torch.bfloat16):
        assert_same(one(inp, g, gl, gh, dt, workspace=small), one(inp, g, gl, gh, dt), f"{dt}")


def test_microbatch_1024_against_the_oracle(orc):
    inp = W.make_inputs(W.MICROBATCH_1024, DEV)
    g, gl, gh = upstream(inp.wl.num_tokens, 11)
    logp, lse, ent, d = one(inp, g, gl, gh, torch.float32)
    inp.grad = g
    stats = P.stream_parity(orc, inp, logp, lse, ent=ent, d=d, g_lse=gl, g_ent=gh, block=256,
                            tag="mb1024 one launch extended")
    print(stats, flush=True)


def test_large_32k_bitwise_and_full_parity(orc):
    """The 32768-row workload: bitwise the two extended calls, and every row's logp,
    LSE, entropy and bf16 dX against the oracle."""
    wl = W.LARGE_32K
    inp = W.make_inputs(wl, DEV)
    g, gl, gh = upstream(wl.num_tokens, 12)
    out = one(inp, g, gl, gh, torch.bfloat16)
    ref = two(inp, g, gl, gh, torch.bfloat16)
    assert_same(out, ref, "32k")
    del ref
    torch.cuda.empty_cache()
    inp.grad = g
    stats = P.stream_parity(orc, inp, out[0], out[1], ent=out[2], d=out[3], g_lse=gl, g_ent=gh,
                            block=1024, tag="32k one launch extended")
    print(stats, flush=True)


@pytest.mark.parametrize("units", [True, False])
def test_validate_reports_data_errors(units):
    wl = W.small_workload(12, 5000, 5008, mask_keep=None, ignore_frac=0.0, num_tiles=64, seed=13)
    inp = W.make_inputs(wl, DEV)
    d = desc_of(wl)
    nbytes = (rlk.rlk_logp_fwd_bwd_ex_workspace_bytes(d) if units
              else rlk.rlk_logp_ex_workspace_bytes(d))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    g, gl, gh = upstream(12, 6)
    one(inp, g, gl, gh, torch.float32, workspace=ws, validate=True)  # clean inputs pass
    inp.targets[3] = 5003  # a padded column: out of range
    with pytest.raises(rlk.RlkError) as ei:
        one(inp, g, gl, gh, torch.float32, workspace=ws, validate=True)
    assert ei.value.status == rlk.RLK_ERR_TARGET_RANGE
    inp.targets[3] = 7
    inp.logits[5, :] = float("-inf")
    with pytest.raises(rlk.RlkError) as ei:
        one(inp, g, gl, gh, torch.float32, workspace=ws, validate=True)
    assert ei.value.status == rlk.RLK_ERR_NONFINITE_LSE
