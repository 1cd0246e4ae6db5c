"""GPU parity of the fused LM-head variant against the oracle (z = h . W^T in
fp64, then the full-vocabulary log-softmax).  Needs an MI355X."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import vocab_selected_token_amd as rlk
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")
IGNORE = -100


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def make_case(n, k, v_real, v_pad, seed, w_sigma=0.05, mask_keep=0.8, ignore_frac=0.1):
    g = torch.Generator(device=DEV).manual_seed(seed)
    h = torch.randn((n, k), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn((v_pad, k), generator=g, device=DEV) * w_sigma).to(torch.bfloat16)
    if v_pad > v_real:  # padding rows hold garbage, and must never be read
        w[v_real:] = torch.randint(-32768, 32768, (v_pad - v_real, k), generator=g, device=DEV,
                                   dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    tgt = torch.randint(0, v_real, (n,), generator=g, device=DEV, dtype=torch.int32)
    mask = torch.rand(n, generator=g, device=DEV) < mask_keep
    tgt[torch.rand(n, generator=g, device=DEV) < ignore_frac] = IGNORE
    return h, w, tgt, mask


def run(h, w, tgt, mask, v_real, v_pad, tiles, validate=False, shards=1):
    n, k = h.shape
    desc = rlk.make_desc(n, v_real, v_pad, v_pad, tiles, shards, IGNORE, validate)
    ws = torch.empty(rlk.rlk_logp_fused_lmhead_workspace_bytes(desc), dtype=torch.uint8,
                     device=DEV)
    logp = torch.empty(n, device=DEV)
    lse = torch.empty(n, device=DEV)
    rlk.rlk_logp_fused_lmhead(desc, h, w, k, tgt, None if mask is None else mask.view(torch.uint8),
                              logp, lse, ws)
    torch.cuda.synchronize()
    return logp, lse, ws


def draw_cases(count: int, seed: int):
    """Seeded ragged shapes: tiles at least 256 columns wide, K a multiple of 64."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        v_real = int(rng.integers(256, 7000))
        v_pad = v_real + int(rng.choice([0, 0, 5, 64, 300]))
        tiles = int(rng.integers(1, v_pad // 256 + 1))
        out.append(dict(n=int(rng.choice([1, 31, 255, 256, 257, 700])),
                        k=int(rng.choice([64, 128, 256, 448])), v_real=v_real, v_pad=v_pad,
                        tiles=tiles))
    return out


CASES = [
    dict(n=37, k=64, v_real=1000, v_pad=1024, tiles=4),
    dict(n=300, k=128, v_real=2500, v_pad=2560, tiles=10),
    dict(n=257, k=320, v_real=3000, v_pad=3000, tiles=7),
    dict(n=1, k=64, v_real=256, v_pad=256, tiles=1),
    dict(n=513, k=192, v_real=5000, v_pad=5120, tiles=3),
] + draw_cases(10, seed=4242)


@pytest.mark.parametrize("c", CASES, ids=lambda c: "n{n}_k{k}_v{v_real}_p{v_pad}_T{tiles}".format(**c))
def test_fused_small_parity(c):
    print(f"case {c}", flush=True)
    h, w, tgt, mask = make_case(c["n"], c["k"], c["v_real"], c["v_pad"], seed=c["n"])
    logp, lse, ws = run(h, w, tgt, mask, c["v_real"], c["v_pad"], c["tiles"])
    o = oracle.get()
    hb, wb = bf16_bits(h), bf16_bits(w)
    z = o.lmhead_logits(hb, wb, real_vocab=c["v_real"])
    t_h, m_h = tgt.cpu().numpy(), mask.cpu().numpy()
    lo, so, _, _ = o.fwd(z, t_h, m_h, real_vocab=c["v_real"])
    act = P.effective_active(t_h, m_h)
    P.check_fwd(logp.cpu().numpy(), lse.cpu().numpy(), lo, so, act, str(c))
    # per-tile partials sit where the materialised path puts them
    n, t = c["n"], c["tiles"]
    part = (n * t * 4 + 255) // 256 * 256
    pm = ws[256:256 + n * t * 4].view(torch.float32).view(n, t).double().cpu().numpy()
    ps = ws[256 + part:256 + part + n * t * 4].view(torch.float32).view(n, t).double().cpu().numpy()
    zp = np.full((n, c["v_pad"]), np.nan)  # padded columns never count
    zp[:, :c["v_real"]] = z
    om, os_ = o.tile_partials(zp, real_vocab=c["v_real"], padded_vocab=c["v_pad"], num_tiles=t)
    ident = om == -np.inf
    assert (pm[ident] == -np.inf).all() and (ps[ident] == 0.0).all()
    assert np.max(np.abs(pm[~ident] - om[~ident])) <= 1e-4
    rel = np.abs(ps[~ident] * np.exp(pm[~ident] - om[~ident]) - os_[~ident]) / os_[~ident]
    assert rel.max() <= 1e-4, rel.max()
    # the target logit is the fp32 accumulator: logp + LSE recovers z[target]
    ztg = z[np.arange(n), np.where(act, t_h, 0)]
    rec = logp.double().cpu().numpy() + lse.double().cpu().numpy()
    assert np.max(np.abs(rec[act] - ztg[act])) <= 1e-4


def partials(ws, n, t):
    """The per-tile (max, sumexp) the fused call leaves in its workspace, as int32 bits."""
    part = (n * t * 4 + 255) // 256 * 256
    return (ws[256:256 + n * t * 4].view(torch.int32).cpu(),
            ws[256 + part:256 + part + n * t * 4].view(torch.int32).cpu())


SHARD_CASES = [
    # 320-column tiles: most shard bounds cut a 256-column GEMM block
    dict(n=300, k=128, v_real=5000, v_pad=5120, tiles=16, shards=[2, 3, 4, 5, 7, 8, 16]),
    # 256-column tiles, real columns end in tile 2: shards of padding only
    dict(n=37, k=64, v_real=700, v_pad=4096, tiles=16, shards=[2, 4, 8, 16]),
    # 428/429-column tiles; the real columns end inside the block a shard bound cuts
    dict(n=257, k=192, v_real=2900, v_pad=3000, tiles=7, shards=[2, 3, 7]),
    # 2384-column tiles as in the 152576-column vocabulary, at a small scale
    dict(n=65, k=64, v_real=18500, v_pad=19072, tiles=8, shards=[2, 4, 8]),
]


@pytest.mark.parametrize("c", SHARD_CASES,
                         ids=lambda c: "n{n}_k{k}_v{v_real}_p{v_pad}_T{tiles}".format(**c))
def test_fused_virtual_shards_bitwise(c):
    """Any grouping of the tiles into virtual shards gives the same bits: logp, LSE
    and every per-tile partial.  Each shard's launches read only its own weight rows
    (the rest hold garbage here), and the result still matches the oracle."""
    print(f"case {c}", flush=True)
    n, t = c["n"], c["tiles"]
    h, w, tgt, mask = make_case(n, c["k"], c["v_real"], c["v_pad"], seed=n + 1000)
    ref = run(h, w, tgt, mask, c["v_real"], c["v_pad"], t)
    ref_bits = (ref[0].view(torch.int32).cpu(), ref[1].view(torch.int32).cpu()) + \
        partials(ref[2], n, t)
    bounds = [(i * c["v_pad"]) // t for i in range(t + 1)]
    for s in c["shards"]:
        got = run(h, w, tgt, mask, c["v_real"], c["v_pad"], t, shards=s)
        got_bits = (got[0].view(torch.int32).cpu(), got[1].view(torch.int32).cpu()) + \
            partials(got[2], n, t)
        for name, a, b in zip(("logp", "lse", "pmax", "psum"), ref_bits, got_bits):
            assert torch.equal(a, b), f"{name} differs at S={s}"
        # the shard that owns the last real column ends there: spoil every weight row
        # past the first shard and check that shard 0's partials do not move
        first_end = bounds[t // s]
        if first_end < c["v_real"]:
            w2 = w.clone()
            w2[first_end:] = torch.randint(-32768, 32768, w2[first_end:].shape, device=DEV,
                                           dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
            spoiled = run(h, w2, tgt, mask, c["v_real"], c["v_pad"], t, shards=s)
            pm_a, ps_a = partials(got[2], n, t)
            pm_b, ps_b = partials(spoiled[2], n, t)
            k0 = t // s  # tiles of shard 0
            assert torch.equal(pm_a.view(n, t)[:, :k0], pm_b.view(n, t)[:, :k0])
            assert torch.equal(ps_a.view(n, t)[:, :k0], ps_b.view(n, t)[:, :k0])
    o = oracle.get()
    z = o.lmhead_logits(bf16_bits(h), bf16_bits(w), real_vocab=c["v_real"])
    t_h, m_h = tgt.cpu().numpy(), mask.cpu().numpy()
    lo, so, _, _ = o.fwd(z, t_h, m_h, real_vocab=c["v_real"])
    P.check_fwd(ref[0].cpu().numpy(), ref[1].cpu().numpy(), lo, so,
                P.effective_active(t_h, m_h), str(c))


def draw_shard_cases(count: int, seed: int):
    """Seeded ragged shapes for the virtual-shard check: tokens 1-513, K of 64-192,
    256-9000 real columns, 0-1000 padded weight rows of random bits, two to five
    shard counts up to T."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        v_real = int(rng.integers(256, 9001))
        v_pad = v_real + int(rng.integers(0, 1001))
        tiles = int(rng.integers(1, v_pad // 256 + 1))
        shards = sorted({int(x) for x in rng.integers(1, tiles + 1, size=int(rng.integers(2, 6)))})
        out.append(dict(i=i, n=int(rng.integers(1, 514)), k=int(rng.choice([64, 128, 192])),
                        v_real=v_real, v_pad=v_pad, tiles=tiles, shards=shards))
    return out


# RLK_LMHEAD_SHARD_SWEEP=80 runs the longer sweep the design notes quote
SHARD_SWEEP = draw_shard_cases(int(os.environ.get("RLK_LMHEAD_SHARD_SWEEP", "12")), seed=8080)


@pytest.mark.parametrize("c", SHARD_SWEEP,
                         ids=lambda c: "{i}_n{n}_k{k}_v{v_real}_p{v_pad}_T{tiles}".format(**c))
def test_fused_virtual_shards_sweep(c):
    """Every drawn shard count gives the bits of S = 1: logp, LSE and every partial;
    and S = 1 matches the oracle (its blocks are cut by tile bounds and the end of
    the real vocabulary wherever the drawn shape puts them)."""
    print(f"case {c}", flush=True)
    n, t = c["n"], c["tiles"]
    h, w, tgt, mask = make_case(n, c["k"], c["v_real"], c["v_pad"], seed=9000 + c["i"])
    ref = run(h, w, tgt, mask, c["v_real"], c["v_pad"], t)
    o = oracle.get()
    z = o.lmhead_logits(bf16_bits(h), bf16_bits(w), real_vocab=c["v_real"])
    t_h, m_h = tgt.cpu().numpy(), mask.cpu().numpy()
    lo, so, _, _ = o.fwd(z, t_h, m_h, real_vocab=c["v_real"])
    P.check_fwd(ref[0].cpu().numpy(), ref[1].cpu().numpy(), lo, so,
                P.effective_active(t_h, m_h), str(c))
    ref_bits = (ref[0].view(torch.int32).cpu(), ref[1].view(torch.int32).cpu()) + \
        partials(ref[2], n, t)
    for s in c["shards"]:
        got = run(h, w, tgt, mask, c["v_real"], c["v_pad"], t, shards=s)
        got_bits = (got[0].view(torch.int32).cpu(), got[1].view(torch.int32).cpu()) + \
            partials(got[2], n, t)
        for name, a, b in zip(("logp", "lse", "pmax", "psum"), ref_bits, got_bits):
            assert torch.equal(a, b), f"{name} differs at S={s}"


def test_fused_repeat_and_batch_invariance():
    h, w, tgt, mask = make_case(300, 128, 2500, 2560, seed=3)
    a = run(h, w, tgt, mask, 2500, 2560, 10)
    b = run(h, w, tgt, mask, 2500, 2560, 10)
    assert torch.equal(a[0].view(torch.int32), b[0].view(torch.int32))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))
    for r in (0, 129, 299):  # a token's result does not depend on the batch
        one = run(h[r:r + 1].contiguous(), w, tgt[r:r + 1], mask[r:r + 1], 2500, 2560, 10)
        assert one[0].view(torch.int32)[0] == a[0].view(torch.int32)[r]
        assert one[1].view(torch.int32)[0] == a[1].view(torch.int32)[r]


def test_fused_validate_bad_target():
    h, w, tgt, mask = make_case(40, 64, 1000, 1024, seed=5, mask_keep=1.1, ignore_frac=0.0)
    tgt[7] = 1000  # a padded column is not a valid target
    for shards in (1, 2, 4):
        with pytest.raises(rlk.RlkError) as ei:
            run(h, w, tgt, None, 1000, 1024, 4, validate=True, shards=shards)
        assert ei.value.status == rlk.RLK_ERR_TARGET_RANGE
        logp, _, _ = run(h, w, tgt, None, 1000, 1024, 4, shards=shards)
        assert torch.isnan(logp[7])
        assert torch.isfinite(logp[torch.arange(40, device=DEV) != 7]).all()


def test_fused_lmhead_4096_full():
    """The LM-head workload: hidden [4096, 4096] ~ N(0,1), W [152576, 4096] ~ N(0, 0.02^2),
    rows >= 151936 padding, 64 tiles, all tokens active; every token against the oracle
    (z = h . W^T in fp64 by matrix product, in blocks of 512 tokens, then the fp64
    log-softmax)."""
    n, k, v_real, v_pad = 4096, 4096, 151936, 152576
    g = torch.Generator(device=DEV).manual_seed(123)
    h = torch.randn((n, k), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn((v_pad, k), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    tgt = torch.randint(0, v_real, (n,), generator=g, device=DEV, dtype=torch.int32)
    logp, lse, _ = run(h, w, tgt, None, v_real, v_pad, 64)
    o = oracle.get()
    wb = bf16_bits(w)
    hb = bf16_bits(h)
    t_all = tgt.cpu().numpy()
    lp_all, ls_all = logp.cpu().numpy(), lse.cpu().numpy()
    worst = {"lse_max_abs": 0.0, "logp_max_abs": 0.0}
    for r0 in range(0, n, 512):
        r1 = min(n, r0 + 512)
        z = o.lmhead_logits_blas(hb[r0:r1], wb, real_vocab=v_real)
        lo, so, _, _ = o.fwd(z, t_all[r0:r1], None, real_vocab=v_real, nthreads=P.host_threads())
        st = P.check_fwd(lp_all[r0:r1], ls_all[r0:r1], lo, so, np.ones(r1 - r0, bool),
                         f"lmhead 4096 tokens {r0}:{r1}")
        worst = {kk: max(worst[kk], st[kk]) for kk in worst}
        del z
    print(worst, flush=True)
    # the 64 tiles grouped into 2, 4 and 8 virtual shards: the same bits
    for s in (2, 4, 8):
        lp_s, lse_s, _ = run(h, w, tgt, None, v_real, v_pad, 64, shards=s)
        assert torch.equal(lp_s.view(torch.int32), logp.view(torch.int32)), s
        assert torch.equal(lse_s.view(torch.int32), lse.view(torch.int32)), s
