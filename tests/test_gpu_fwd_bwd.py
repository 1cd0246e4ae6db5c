"""GPU parity of the one-launch forward+backward (rlk_logp_fwd_bwd).

Two bars, both through the C ABI:
  * against the CPU oracle, to the same tolerances as the separate calls
    (LSE and logp 1e-4, fp32 dX 1e-5, bf16 dX one bf16 spacing / 8e-3, inactive
    rows and padded columns +0 bit for bit);
  * bit for bit against rlk_logp_fwd followed by rlk_logp_bwd on the same
    inputs, since the one-launch schedule computes every value with the same
    arithmetic in the same order.
Inputs come from workloads.py (seeded, synthetic).
"""
from __future__ import annotations

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


def fused(inp, dtype, shards=1, validate=False, mask="wl"):
    wl = inp.wl
    m = inp.mask if mask == "wl" else mask
    return rlk.forward_backward(inp.logits, inp.targets, m, inp.grad, real_vocab=wl.real_vocab,
                                padded_vocab=wl.padded_vocab, num_vocab_tiles=wl.num_tiles,
                                num_virtual_shards=shards, out_dtype=dtype, validate=validate)


def separate(inp, dtype, shards=1):
    wl = inp.wl
    logp, lse = rlk.forward(inp.logits, inp.targets, inp.mask, real_vocab=wl.real_vocab,
                            padded_vocab=wl.padded_vocab, num_vocab_tiles=wl.num_tiles,
                            num_virtual_shards=shards)
    d = rlk.backward(inp.logits, inp.targets, inp.mask, lse, inp.grad, real_vocab=wl.real_vocab,
                     padded_vocab=wl.padded_vocab, out_dtype=dtype, num_vocab_tiles=wl.num_tiles)
    return logp, lse, d


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def assert_same_bits(a, b, what):
    for x, y, name in zip(a, b, ("logp", "lse", "dlogits")):
        assert torch.equal(bits(x), bits(y)), f"{what}: {name} differs from the separate calls"


def raw_bits(d: torch.Tensor) -> np.ndarray:
    if d.dtype == torch.bfloat16:
        return d.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return d.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def check_oracle(orc, inp, out, dtype, tag, rows=None):
    """out = (logp, lse, dlogits) of the whole batch; rows = sampled rows or None."""
    wl = inp.wl
    logp, lse, d = out
    host = W.to_host(inp, rows)
    xb, tgt, mask, g = host
    act = P.effective_active(tgt, mask)
    lo, so, _, _ = orc.fwd(xb, tgt, mask, real_vocab=wl.real_vocab, raise_on_error=False)
    sel = slice(None) if rows is None else torch.from_numpy(rows).to(DEV)
    P.check_fwd(logp[sel].cpu().numpy(), lse[sel].cpu().numpy(), lo, so, act, tag)
    ds = d[sel]
    dg, rb = P.dlogits_host(ds), raw_bits(ds)
    blk = 256
    for r0 in range(0, len(tgt), blk):
        r1 = min(len(tgt), r0 + blk)
        do = orc.bwd(xb[r0:r1], tgt[r0:r1], mask[r0:r1], so[r0:r1], g[r0:r1],
                     real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab, raise_on_error=False)
        P.check_bwd(dg[r0:r1], do, act[r0:r1], wl.real_vocab, dtype == torch.bfloat16,
                    f"{tag} rows {r0}:{r1}", rb[r0:r1])


SMALL = [
    dict(n=37, real=1000, pad=1000, T=7),
    dict(n=64, real=5000, pad=5120, ld=5128, T=64),
    dict(n=16, real=100, pad=128, T=8),
    dict(n=5, real=1, pad=8, T=1),
    dict(n=3, real=17, pad=17, T=17),
    dict(n=130, real=151936, pad=152576, T=64),
    dict(n=9, real=3001, pad=3008, T=5, spike=True),
    dict(n=33, real=2374 * 3 + 1, pad=2374 * 3 + 8, T=3),
    # more tiles than a wave has lanes: the merge reads the partials from LDS
    dict(n=21, real=9000, pad=9000, T=65),
    dict(n=12, real=30000, pad=30008, T=100),
    dict(n=6, real=4000, pad=4096, T=1024),
    # fewer columns than tiles would leave whole tiles empty
    dict(n=4, real=300, pad=1024, T=1024),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"n{c['n']}_v{c['real']}_p{c['pad']}_T{c['T']}")
def test_small_parity_and_bitwise_equality(orc, case):
    print(f"case {case}", flush=True)
    wl = W.small_workload(case["n"], case["real"], case["pad"], ld=case.get("ld"),
                          num_tiles=case["T"], spike_frac=0.3 if case.get("spike") else 0.0,
                          spike=12.0, seed=case["n"] + 1000)
    inp = W.make_inputs(wl, DEV)
    for dt in (torch.float32, torch.bfloat16):
        out = fused(inp, dt)
        check_oracle(orc, inp, out, dt, f"{case} {dt}")
        assert_same_bits(out, separate(inp, dt), f"{case} {dt}")
        for s in sorted({2, 8, case["T"]} & set(range(2, case["T"] + 1))):
            assert_same_bits(fused(inp, dt, shards=s), out, f"{case} {dt} S={s}")


# Larger batches of ragged shapes, with T above 64 (the merge from LDS),
# all-padding tiles and rows without a finite logit or holding a NaN.
LARGER = [
    dict(n=1024, real=1000, pad=1000, T=7),
    dict(n=1031, real=5000, pad=5120, ld=5128, T=64),
    dict(n=1300, real=9000, pad=9000, T=65),
    dict(n=1500, real=4000, pad=4096, T=1024),
    dict(n=1029, real=300, pad=1024, T=1024),
    dict(n=2100, real=2374 * 3 + 1, pad=2374 * 3 + 8, T=3, spike=True),
]


@pytest.mark.parametrize("case", LARGER, ids=lambda c: f"n{c['n']}_v{c['real']}_p{c['pad']}_T{c['T']}")
def test_larger_batches_parity_and_bitwise_equality(orc, case):
    print(f"case {case}", flush=True)
    wl = W.small_workload(case["n"], case["real"], case["pad"], ld=case.get("ld"),
                          num_tiles=case["T"], spike_frac=0.3 if case.get("spike") else 0.0,
                          spike=12.0, seed=case["n"] + 3000)
    inp = W.make_inputs(wl, DEV)
    inp.logits[5, :wl.real_vocab] = float("-inf")  # no finite logit: LSE -inf
    inp.logits[6, min(3, wl.real_vocab - 1)] = float("nan")
    inp.mask[5] = False
    inp.mask[6] = False
    for dt in (torch.float32, torch.bfloat16):
        out = fused(inp, dt)
        ref = separate(inp, dt)
        for a, b, name in zip(out, ref, ("logp", "lse", "dlogits")):
            na, nb = torch.isnan(a), torch.isnan(b)
            assert torch.equal(na, nb), f"{case} {dt} {name}: NaN pattern differs"
            assert torch.equal(bits(a)[~na], bits(b)[~nb]), f"{case} {dt} {name}: bits differ"
        keep = torch.ones(wl.num_tokens, dtype=torch.bool, device=DEV)
        keep[5:7] = False
        rows = torch.nonzero(keep).flatten().cpu().numpy()
        check_oracle(orc, inp, out, dt, f"{case} {dt}", rows=rows)
        for s in sorted({2, 8, case["T"]} & set(range(2, case["T"] + 1))):
            o2 = fused(inp, dt, shards=s)
            for a, b, name in zip(o2, out, ("logp", "lse", "dlogits")):
                na = torch.isnan(a)
                assert torch.equal(na, torch.isnan(b)) and torch.equal(bits(a)[~na],
                                                                      bits(b)[~na]), f"S={s} {name}"


# Geometries the unit schedule takes (T <= 64, tiles of 8 to about 2,500
# columns): full-size tiles of four passes, tile bounds off the 8-column grid,
# a last unit with fewer than 4 tiles, 8- and 9-column tiles, a real vocabulary
# ending inside a chunk, whole tiles of padding, one tile per row.
UNIT_SHAPES = [
    dict(n=300, real=151936, pad=152576, T=64),
    dict(n=64, real=5000, pad=5120, ld=5128, T=64),
    dict(n=9, real=3001, pad=3008, T=5, spike=True),
    dict(n=33, real=2374 * 3 + 1, pad=2374 * 3 + 8, T=3),
    dict(n=40, real=500, pad=512, T=64),
    dict(n=40, real=515, pad=600, T=64),
    dict(n=20, real=700, pad=2048, T=64),
    dict(n=17, real=1, pad=8, T=1),
    dict(n=50, real=2504, pad=2504, T=1),
    dict(n=1100, real=9000, pad=9001, T=61),
]


def rows_schedule(inp, dtype):
    """forward_backward with only the status words as workspace: one block per row."""
    wl = inp.wl
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    return rlk.forward_backward(inp.logits, inp.targets, inp.mask, inp.grad,
                                real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab,
                                num_vocab_tiles=wl.num_tiles, out_dtype=dtype, workspace=ws)


def assert_same_bits_nan(a3, b3, what):
    for a, b, name in zip(a3, b3, ("logp", "lse", "dlogits")):
        na, nb = torch.isnan(a), torch.isnan(b)
        assert torch.equal(na, nb), f"{what} {name}: NaN pattern differs"
        assert torch.equal(bits(a)[~na], bits(b)[~nb]), f"{what} {name}: bits differ"


@pytest.mark.parametrize("case", UNIT_SHAPES,
                         ids=lambda c: f"n{c['n']}_v{c['real']}_p{c['pad']}_T{c['T']}")
def test_unit_schedule_matches_row_schedule(case):
    """Where the geometry fits, rlk_logp_fwd_bwd with its full workspace runs the
    unit schedule (blocks of 8 tiles that exchange partials); with only the
    status words it runs one block per row.  Both give the bits of the separate
    calls, on rows with NaN, +inf and no finite logit too."""
    print(f"case {case}", flush=True)
    wl = W.small_workload(case["n"], case["real"], case["pad"], ld=case.get("ld"),
                          num_tiles=case["T"], spike_frac=0.3 if case.get("spike") else 0.0,
                          spike=12.0, seed=case["n"] + 5000)
    d = rlk.make_desc(wl.num_tokens, wl.real_vocab, wl.padded_vocab, wl.ld_logits, wl.num_tiles)
    assert rlk.rlk_logp_fwd_bwd_workspace_bytes(d) == 256 + 8 * wl.num_tokens * wl.num_tiles
    inp = W.make_inputs(wl, DEV)
    n = wl.num_tokens
    if n > 6:
        inp.logits[1, :wl.real_vocab] = float("-inf")
        inp.logits[2, wl.real_vocab - 1] = float("nan")
        inp.logits[3, 0] = float("inf")
        inp.mask[1] = True
        inp.targets[4] = wl.real_vocab + 3  # a bad target on an active row
        inp.mask[4] = True
    if n > 6:
        # a bf16 NaN with every payload bit set: the largest-payload tile max there
        # is (0xFFFF0000 widened), which must still differ from the empty-slot
        # sentinel
        inp.logits[5].view(torch.int16)[wl.real_vocab // 2] = -1
    ws = torch.empty(rlk.rlk_logp_fwd_bwd_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    for dt in (torch.float32, torch.bfloat16):
        units = rlk.forward_backward(inp.logits, inp.targets, inp.mask, inp.grad,
                                     real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab,
                                     num_vocab_tiles=wl.num_tiles, out_dtype=dt, workspace=ws)
        torch.cuda.synchronize()
        # status word 2: no block had to compute its row's partials itself
        assert ws[:12].view(torch.int32)[2].item() == 0, f"{case} {dt}: exchange fell back"
        assert_same_bits_nan(units, rows_schedule(inp, dt), f"{case} {dt} units vs rows")
        assert_same_bits_nan(units, separate(inp, dt), f"{case} {dt} units vs separate")


def test_empty_batch():
    wl = W.small_workload(0, 100)
    inp = W.make_inputs(wl, DEV)
    logp, lse, d = fused(inp, torch.float32)
    assert logp.numel() == 0 and lse.numel() == 0 and d.shape == (0, 100)


def test_matrix_b2s16_full(orc):
    inp = W.make_inputs(W.MATRIX_B2S16, DEV)
    out = fused(inp, torch.float32)
    check_oracle(orc, inp, out, torch.float32, "matrix_b2s16")
    assert_same_bits(out, separate(inp, torch.float32), "matrix_b2s16")


def test_microbatch_1024_full(orc):
    inp = W.make_inputs(W.MICROBATCH_1024, DEV)
    out = fused(inp, torch.float32)
    check_oracle(orc, inp, out, torch.float32, "microbatch_1024")
    assert_same_bits(out, separate(inp, torch.float32), "microbatch_1024")


def test_large_32k_bitwise_and_full_parity(orc):
    """The one launch on the 32768-row workload: bitwise the two calls, and every
    row's LSE, logp and bf16 dX against the oracle."""
    wl = W.LARGE_32K
    inp = W.make_inputs(wl, DEV)
    out = fused(inp, torch.bfloat16)
    ref = separate(inp, torch.bfloat16)
    assert_same_bits(out, ref, "32k")
    del ref
    torch.cuda.empty_cache()
    stats = P.stream_parity(orc, inp, out[0], out[1], d=out[2], block=1024, tag="32k one launch")
    print(stats, flush=True)


def test_repeats_and_batch_invariance():
    wl = W.small_workload(48, 151936, 152576, seed=21)
    inp = W.make_inputs(wl, DEV)
    ref = fused(inp, torch.bfloat16)
    for _ in range(3):
        assert_same_bits(fused(inp, torch.bfloat16), ref, "repeat")
    for r in (0, 29, 47):
        sub = W.Inputs(wl, inp.logits[r:r + 1], inp.targets[r:r + 1], inp.mask[r:r + 1],
                       inp.grad[r:r + 1])
        one = fused(sub, torch.bfloat16)
        assert_same_bits(one, tuple(t[r:r + 1] for t in ref), f"row {r} alone")


def test_validate_reports_data_errors():
    wl = W.small_workload(12, 5000, 5008, mask_keep=None, ignore_frac=0.0, seed=9)
    inp = W.make_inputs(wl, DEV)
    base = fused(inp, torch.float32)
    m = torch.ones(12, dtype=torch.bool, device=DEV)
    m[3] = False
    inp.targets[3] = 10 ** 9
    fused(inp, torch.float32, validate=True, mask=m)  # inactive rows may hold any target
    for bad in (-1, 5000, 5007, 10 ** 9):
        inp.targets[3] = bad
        with pytest.raises(rlk.RlkError) as ei:
            fused(inp, torch.float32, validate=True)
        assert ei.value.status == rlk.RLK_ERR_TARGET_RANGE
        logp, lse, d = fused(inp, torch.float32)
        assert torch.isnan(logp[3]) and torch.equal(lse, base[1])
        keep = torch.arange(12, device=DEV) != 3
        assert torch.equal(bits(logp[keep]), bits(base[0][keep]))
        assert torch.isnan(d[3, :5000]).all() and (bits(d[3, 5000:]) == 0).all()
        assert torch.equal(bits(d[keep]), bits(base[2][keep]))
    inp.targets[3] = 7
    inp.logits[5, :] = float("-inf")
    with pytest.raises(rlk.RlkError) as ei:
        fused(inp, torch.float32, validate=True)
    assert ei.value.status == rlk.RLK_ERR_NONFINITE_LSE
    m = torch.ones(12, dtype=torch.bool, device=DEV)
    m[5] = False
    logp, lse, d = fused(inp, torch.float32, validate=True, mask=m)
    assert lse[5].item() == float("-inf") and (bits(d[5]) == 0).all()


def test_side_stream():
    wl = W.small_workload(50, 20000, 20000, seed=4)
    inp = W.make_inputs(wl, DEV)
    ref = fused(inp, torch.float32)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = fused(inp, torch.float32)
    s.synchronize()
    assert_same_bits(out, ref, "side stream")


def test_nonfinite_logits_match_separate_calls(orc):
    """NaN, +inf and -inf among the real logits: the one-launch outputs agree with
    the separate calls (NaN where they are NaN, bits elsewhere) and with the oracle."""
    wl = W.small_workload(24, 151936, 152576, mask_keep=None, ignore_frac=0.0, seed=31)
    inp = W.make_inputs(wl, DEV)
    inp.logits[0, 100] = float("nan")
    inp.logits[1, 7] = float("inf")
    inp.logits[2, :] = float("-inf")
    inp.logits[3, :50000] = float("-inf")
    inp.logits[4, 151935] = float("nan")
    m = torch.ones(24, dtype=torch.bool, device=DEV)
    m[0] = False  # an inactive NaN row: LSE NaN, logp +0, dX +0
    for dt in (torch.float32, torch.bfloat16):
        out = fused(inp, dt, mask=m)
        ref = rlk.forward(inp.logits, inp.targets, m, real_vocab=wl.real_vocab,
                          padded_vocab=wl.padded_vocab, num_vocab_tiles=wl.num_tiles)
        ref = ref + (rlk.backward(inp.logits, inp.targets, m, ref[1], inp.grad,
                                  real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab,
                                  out_dtype=dt, num_vocab_tiles=wl.num_tiles),)
        for a, b, name in zip(out, ref, ("logp", "lse", "dlogits")):
            na, nb = torch.isnan(a), torch.isnan(b)
            assert torch.equal(na, nb), f"{dt} {name}: NaN pattern differs"
            assert torch.equal(bits(a)[~na], bits(b)[~nb]), f"{dt} {name}: bits differ"
        xb, tgt, mask, _ = W.to_host(inp)
        mask = m.cpu().numpy()
        lo, so, _, _ = orc.fwd(xb, tgt, mask, real_vocab=wl.real_vocab, raise_on_error=False)
        lse = out[1].double().cpu().numpy()
        assert np.array_equal(np.isnan(lse), np.isnan(so))
        assert np.array_equal(np.isinf(lse), np.isinf(so))
        assert (bits(out[2][0]) == 0).all() and bits(out[0][:1]).item() == 0
