"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every test here needs an MI355X.  Inputs come from workloads.py (seeded,
synthetic); the oracle reads host copies of the very same tensors.  Every
case, the benchmark-sized workloads included, is compared row by row in full;
the large ones are streamed through the oracle in row blocks so that host
memory stays bounded.
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


def fwd(inp, shards=1, validate=False, num_tiles=None, mask="wl"):
    wl = inp.wl
    m = inp.mask if mask == "wl" else mask
    return rlk.forward(inp.logits, inp.targets, m, real_vocab=wl.real_vocab,
                       padded_vocab=wl.padded_vocab, num_vocab_tiles=num_tiles or wl.num_tiles,
                       num_virtual_shards=shards, validate=validate)


def bwd(inp, lse, dtype, validate=False):
    wl = inp.wl
    return rlk.backward(inp.logits, inp.targets, inp.mask, lse, inp.grad,
                        real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab, out_dtype=dtype,
                        validate=validate, num_vocab_tiles=wl.num_tiles)


def raw_bits(d: torch.Tensor) -> np.ndarray:
    if d.dtype == torch.bfloat16:
        return d.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return d.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def oracle_fwd(orc, host, wl):
    bits, tgt, mask, _ = host
    logp, lse, _, _ = orc.fwd(bits, tgt, mask, real_vocab=wl.real_vocab, raise_on_error=False)
    return logp, lse


def check_full(orc, inp, dtypes=(torch.float32, torch.bfloat16), tag=""):
    wl = inp.wl
    host = W.to_host(inp)
    bits, tgt, mask, g = host
    act = P.effective_active(tgt, mask)
    logp, lse = fwd(inp)
    lo, so = oracle_fwd(orc, host, wl)
    stats = P.check_fwd(logp.cpu().numpy(), lse.cpu().numpy(), lo, so, act, tag)
    for dt in dtypes:
        d = bwd(inp, lse, dt)
        dg = P.dlogits_host(d)
        rb = raw_bits(d)
        blk = 256
        for r0 in range(0, wl.num_tokens, blk):
            r1 = min(wl.num_tokens, r0 + blk)
            do = orc.bwd(bits[r0:r1], tgt[r0:r1], mask[r0:r1], so[r0:r1], g[r0:r1],
                         real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab,
                         raise_on_error=False)
            P.check_bwd(dg[r0:r1], do, act[r0:r1], wl.real_vocab, dt == torch.bfloat16,
                        f"{tag} {dt} rows {r0}:{r1}", rb[r0:r1])
    return logp, lse, stats


SMALL = [
    dict(n=37, real=1000, pad=1000, T=7),
    dict(n=64, real=5000, pad=5120, ld=5128, T=64),
    dict(n=16, real=100, pad=128, T=8),
    dict(n=5, real=1, pad=8, T=1),
    dict(n=3, real=17, pad=17, T=17),
    dict(n=300, real=151936, pad=151936, T=64),
    dict(n=130, real=151936, pad=152576, T=64),
    dict(n=7, real=20000, pad=20000, T=1),
    dict(n=9, real=3001, pad=3008, T=5, spike=True),
    dict(n=33, real=2374 * 3 + 1, pad=2374 * 3 + 8, T=3),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"n{c['n']}_v{c['real']}_p{c['pad']}_T{c['T']}")
def test_small_parity_and_regrouping(orc, case):
    print(f"case {case}", flush=True)
    wl = W.small_workload(case["n"], case["real"], case["pad"], ld=case.get("ld"),
                          num_tiles=case["T"], spike_frac=0.3 if case.get("spike") else 0.0,
                          spike=12.0, seed=case["n"])
    inp = W.make_inputs(wl, DEV)
    logp, lse, _ = check_full(orc, inp, tag=str(case))
    # any grouping of the tiles into virtual shards gives identical bits
    for s in sorted({2, 3, 7, case["T"]} & set(range(1, case["T"] + 1))):
        l2, s2 = fwd(inp, shards=s)
        assert torch.equal(l2.view(torch.int32), logp.view(torch.int32)), f"S={s} logp"
        assert torch.equal(s2.view(torch.int32), lse.view(torch.int32)), f"S={s} lse"


def test_empty_batch():
    wl = W.small_workload(0, 100)
    inp = W.make_inputs(wl, DEV)
    logp, lse = fwd(inp)
    assert logp.numel() == 0 and lse.numel() == 0
    d = bwd(inp, lse, torch.float32)
    assert d.shape == (0, 100)


@pytest.mark.parametrize("shape", [(40, 151936, 151936, 64), (24, 3001, 3008, 5),
                                   (16, 100, 128, 8), (8, 20000, 20000, 1)])
def test_stage1_partials_match_oracle(orc, shape):
    """The per-tile statistic itself: exact maxima, sums within 1e-5 relative,
    the (-inf, 0) identity on tiles without real columns."""
    n, real, pad, t = shape
    wl = W.small_workload(n, real, pad, num_tiles=t, seed=5)
    inp = W.make_inputs(wl, DEV)
    inp.logits[1, :real] = float("-inf")  # every tile of row 1 is an identity partial
    desc = rlk.make_desc(n, real, pad, inp.logits.stride(0), t)
    ws = rlk.workspace_for(desc, DEV)
    logp = torch.empty(n, device=DEV)
    lse = torch.empty(n, device=DEV)
    rlk.rlk_logp_fwd(desc, inp.logits, inp.targets, None, logp, lse, ws)
    torch.cuda.synchronize()
    part = (n * t * 4 + 255) // 256 * 256
    pm = ws[256:256 + n * t * 4].view(torch.float32).view(n, t).double().cpu().numpy()
    ps = ws[256 + part:256 + part + n * t * 4].view(torch.float32).view(n, t).double().cpu().numpy()
    bits, _, _, _ = W.to_host(inp)
    om, os_ = orc.tile_partials(bits, real_vocab=real, padded_vocab=pad, num_tiles=t)
    assert np.array_equal(pm, om), "per-tile maxima must be exact"
    ident = om == -np.inf
    assert (ps[ident] == 0.0).all()
    rel = np.abs(ps[~ident] - os_[~ident]) / os_[~ident]
    assert rel.max() <= 1e-5, rel.max()


def test_matrix_b2s16_full(orc):
    inp = W.make_inputs(W.MATRIX_B2S16, DEV)
    logp, lse, stats = check_full(orc, inp, dtypes=(torch.float32,), tag="matrix_b2s16")
    print(stats, flush=True)
    shas = set()
    for s in (1, 2, 4, 8):
        for _ in range(2):
            l2, s2 = fwd(inp, shards=s)
            shas.add((W.sha256(l2), W.sha256(s2)))
    assert len(shas) == 1


def test_microbatch_1024_full(orc):
    inp = W.make_inputs(W.MICROBATCH_1024, DEV)
    _, _, stats = check_full(orc, inp, dtypes=(torch.float32,), tag="microbatch_1024")
    print(stats, flush=True)


def test_throughput_16k_regrouping_and_full_parity(orc):
    """16384 x 151936, forward only: the SHA-256 of logp and LSE is the same at
    S = 1, 2, 4 and 8, and every row matches the oracle (LSE on all rows, logp on
    every active row)."""
    wl = W.THROUGHPUT_16K
    inp = W.make_inputs(wl, DEV)
    outs = {s: fwd(inp, shards=s) for s in wl.shards}
    shas = {s: (W.sha256(l), W.sha256(x)) for s, (l, x) in outs.items()}
    assert len(set(shas.values())) == 1, shas
    logp, lse = outs[1]
    stats = P.stream_parity(orc, inp, logp, lse, block=2048, tag="16k")
    print(stats, flush=True)


def test_large_32k_full_parity(orc):
    """32768 x 152576 (real 151936), bf16 dX: S = 8 gives the bits of S = 1, and every
    row's LSE, logp and dX matches the oracle, whose backward uses its own LSE."""
    wl = W.LARGE_32K
    inp = W.make_inputs(wl, DEV)
    logp, lse = fwd(inp)
    l8, s8 = fwd(inp, shards=8)
    assert torch.equal(l8.view(torch.int32), logp.view(torch.int32))
    assert torch.equal(s8.view(torch.int32), lse.view(torch.int32))
    del l8, s8
    d = bwd(inp, lse, torch.bfloat16)
    stats = P.stream_parity(orc, inp, logp, lse, d=d, block=1024, tag="32k")
    print(stats, flush=True)
    assert stats["rows"] == wl.num_tokens


def test_repeats_batch_invariance_and_padding_invariance():
    wl = W.small_workload(64, 151936, 152576, seed=11)
    inp = W.make_inputs(wl, DEV)
    ref = fwd(inp)
    for _ in range(3):
        again = fwd(inp)
        assert torch.equal(again[0].view(torch.int32), ref[0].view(torch.int32))
        assert torch.equal(again[1].view(torch.int32), ref[1].view(torch.int32))
    # a row's result does not depend on the batch it sits in
    for r in (0, 17, 63):
        sub = W.Inputs(wl, inp.logits[r:r + 1], inp.targets[r:r + 1], inp.mask[r:r + 1],
                       inp.grad[r:r + 1])
        one = fwd(sub)
        assert one[0].view(torch.int32)[0] == ref[0].view(torch.int32)[r]
        assert one[1].view(torch.int32)[0] == ref[1].view(torch.int32)[r]
    # whatever the padding holds, nothing changes
    d_ref = bwd(inp, ref[1], torch.float32)
    for fill in (0.0, float("nan"), float("-inf"), float("inf")):
        x = inp.logits.clone()
        x[:, wl.real_vocab:] = fill
        alt = W.Inputs(wl, x, inp.targets, inp.mask, inp.grad)
        out = fwd(alt)
        assert torch.equal(out[0].view(torch.int32), ref[0].view(torch.int32)), fill
        assert torch.equal(out[1].view(torch.int32), ref[1].view(torch.int32)), fill
        d_alt = bwd(alt, ref[1], torch.float32)
        assert torch.equal(d_alt.view(torch.int32), d_ref.view(torch.int32)), fill


def test_closed_forms_and_exact_gather():
    v = 151936
    n = 8
    wl = W.small_workload(n, v, mask_keep=None, ignore_frac=0.0, seed=3)
    inp = W.make_inputs(wl, DEV)
    cs = [0.0, 1.5, -3.0, 7.25]
    for i, c in enumerate(cs):
        inp.logits[i, :] = c
    # rows 4..7: one finite value a, the rest -inf
    for i, (pos, a) in enumerate(((5, 3.25), (v - 1, -7.5), (75968, 12.0), (2374, 0.5))):
        inp.logits[4 + i, :] = float("-inf")
        inp.logits[4 + i, pos] = a
        inp.targets[4 + i] = pos
    logp, lse = fwd(inp)
    lse_h, logp_h = lse.cpu().numpy(), logp.cpu().numpy()
    for i, c in enumerate(cs):
        assert abs(lse_h[i] - (c + math.log(v))) <= 1e-4
        assert abs(logp_h[i] + math.log(v)) <= 1e-4
    for i, (_, a) in enumerate(((5, 3.25), (v - 1, -7.5), (75968, 12.0), (2374, 0.5))):
        assert lse_h[4 + i] == np.float32(a), (i, lse_h[4 + i], a)
        assert P.f32_bits(logp_h[4 + i:5 + i])[0] == 0  # +0.0
    # the gather is exact: logp is fp32(x[target]) - LSE in one fp32 subtraction
    x_t = inp.logits[torch.arange(n, device=DEV), inp.targets.long()].float().cpu().numpy()
    assert np.array_equal(P.f32_bits(x_t - lse_h), P.f32_bits(logp_h))


def test_validate_reports_data_errors():
    wl = W.small_workload(12, 5000, 5008, mask_keep=None, ignore_frac=0.0, seed=9)
    inp = W.make_inputs(wl, DEV)
    base = fwd(inp)
    # inactive rows may hold any target
    m = torch.ones(12, dtype=torch.bool, device=DEV)
    m[3] = False
    inp.targets[3] = 10 ** 9
    fwd(inp, validate=True, mask=m)
    # an effective-active target outside [0, V_real): error, NaN, no OOB read
    for bad in (-1, 5000, 5007, 10 ** 9):
        inp.targets[3] = bad
        with pytest.raises(rlk.RlkError) as ei:
            fwd(inp, validate=True)
        assert ei.value.status == rlk.RLK_ERR_TARGET_RANGE
        with pytest.raises(rlk.RlkError) as ei:
            bwd(inp, base[1], torch.float32, validate=True)
        assert ei.value.status == rlk.RLK_ERR_TARGET_RANGE
        logp, lse = fwd(inp)
        assert torch.isnan(logp[3])
        keep = torch.arange(12, device=DEV) != 3
        assert torch.equal(logp[keep], base[0][keep]) and torch.equal(lse, base[1])
        d = bwd(inp, lse, torch.float32)
        assert torch.isnan(d[3, :5000]).all() and (d[3, 5000:] == 0).all()
    inp.targets[3] = 7
    # a non-finite LSE on an effective-active row
    inp.logits[5, :] = float("-inf")
    with pytest.raises(rlk.RlkError) as ei:
        fwd(inp, validate=True)
    assert ei.value.status == rlk.RLK_ERR_NONFINITE_LSE
    _, lse = fwd(inp)
    assert lse[5].item() == float("-inf")
    m = torch.ones(12, dtype=torch.bool, device=DEV)
    m[5] = False
    fwd(inp, validate=True, mask=m)  # inactive: returned as is, no error


def test_side_stream():
    wl = W.small_workload(50, 20000, 20000, seed=4)
    inp = W.make_inputs(wl, DEV)
    ref = fwd(inp)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = fwd(inp)
    s.synchronize()
    assert torch.equal(out[0].view(torch.int32), ref[0].view(torch.int32))
    assert torch.equal(out[1].view(torch.int32), ref[1].view(torch.int32))


def test_small_and_large_launch_shapes_agree():
    """Stage 1 packs a small batch into one-wave blocks and a large one into
    four-wave blocks; a row gives the same bits either way (batch invariance
    across the two launch shapes)."""
    wl = W.small_workload(512, 151936, 152576, seed=27)  # 512 x 64 items: four-wave blocks
    inp = W.make_inputs(wl, DEV)
    big = fwd(inp)
    for r0, r1 in ((0, 1), (5, 37), (100, 164), (448, 512)):  # small launches: one-wave blocks
        sub = W.Inputs(wl, inp.logits[r0:r1], inp.targets[r0:r1], inp.mask[r0:r1],
                       inp.grad[r0:r1])
        part = fwd(sub)
        assert torch.equal(part[0].view(torch.int32), big[0][r0:r1].view(torch.int32))
        assert torch.equal(part[1].view(torch.int32), big[1][r0:r1].view(torch.int32))
    # and the same for the entropy statistic
    _, _, e_big = rlk.forward_ex(inp.logits, inp.targets, inp.mask, real_vocab=wl.real_vocab)
    _, _, e_one = rlk.forward_ex(inp.logits[7:8], inp.targets[7:8], inp.mask[7:8],
                                 real_vocab=wl.real_vocab)
    assert torch.equal(e_one.view(torch.int32), e_big[7:8].view(torch.int32))


@pytest.mark.parametrize("tiles", [64, 16])
def test_batch_invariance_across_stage2_forms(tiles):
    """Batches of up to 4096 rows merge with one wave per row, larger ones with one
    thread per row; a row gives the same bits either way, including rows whose
    logits are all -inf, hold a NaN or hold +inf."""
    wl = W.small_workload(5000, 5000, 5120, num_tiles=tiles, sigma=3.0, mask_keep=0.9,
                          ignore_frac=0.05, seed=4096 + tiles)
    inp = W.make_inputs(wl, DEV)
    x = inp.logits
    x[3, :wl.real_vocab] = float("-inf")
    x[10, 77] = float("nan")
    x[20, 4000] = float("inf")
    x[21, :wl.real_vocab] = float("-inf")
    x[21, 123] = 2.5  # one finite value: LSE is exactly that value
    big = fwd(inp)
    rows = torch.tensor(sorted({3, 10, 20, 21} | set(range(0, 5000, 79))), device=DEV)
    assert len(rows) <= 4096
    sub = W.Inputs(wl, x[rows].contiguous(), inp.targets[rows], inp.mask[rows], inp.grad[rows])
    small = fwd(sub)
    assert torch.equal(small[0].view(torch.int32), big[0][rows].view(torch.int32))
    assert torch.equal(small[1].view(torch.int32), big[1][rows].view(torch.int32))
    lse = big[1].cpu()
    assert lse[3] == float("-inf") and torch.isnan(lse[10]) and lse[21] == 2.5
    assert torch.isnan(lse[20]) or lse[20] == float("inf")
    # the same with the entropy output (its own wave-per-row merge)
    kw = dict(real_vocab=wl.real_vocab, padded_vocab=wl.padded_vocab, num_vocab_tiles=tiles)
    big_ex = rlk.forward_ex(x, inp.targets, inp.mask, **kw)
    small_ex = rlk.forward_ex(sub.logits, sub.targets, sub.mask, **kw)
    for a, b in zip(small_ex, big_ex):
        assert torch.equal(a.view(torch.int32), b[rows].view(torch.int32))
    assert torch.equal(big_ex[1].view(torch.int32), big[1].view(torch.int32))
    assert float(big_ex[2][21]) == 0.0  # one finite value: no uncertainty
