"""Every entry point called without RLK_FLAG_VALIDATE enqueues kernel launches
only -- no allocation, no memset, no copy, no synchronisation -- so a caller can
capture it into a HIP graph.  One graph holds a call of each entry point (the
one-launch calls in their unit schedule, whose slot fill is a kernel); it is
replayed several times, with a different input set copied into the captured
buffers before each replay and eager work in between, and every replay must give
the bits of the same calls made eagerly on that input set.  Needs an MI355X."""
from __future__ import annotations

import pytest
import torch

import vocab_selected_token_amd as rlk
import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")
N, V_REAL, V_PAD, TILES, K = 300, 5000, 5120, 16, 128


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).clone()


def make_set(seed: int):
    wl = W.small_workload(N, V_REAL, V_PAD, num_tiles=TILES, sigma=2.0, mask_keep=0.8,
                          ignore_frac=0.05, seed=seed)
    inp = W.make_inputs(wl, DEV)
    gen = torch.Generator(device=DEV).manual_seed(seed + 1)
    h = torch.randn((N, K), generator=gen, device=DEV).to(torch.bfloat16)
    w = (torch.randn((V_PAD, K), generator=gen, device=DEV) * 0.1).to(torch.bfloat16)
    return {"x": inp.logits, "tg": inp.targets, "m": inp.mask.to(torch.uint8), "g": inp.grad,
            "h": h, "w": w}


def test_graph_replays_match_eager():
    sets = [make_set(s) for s in (31, 32, 33)]
    st = {k: torch.empty_like(v) for k, v in sets[0].items()}  # the buffers the graph reads
    gl = torch.linspace(-1.0, 1.0, N, device=DEV)
    gh = torch.full((N,), 0.25, device=DEV)
    d1 = rlk.make_desc(N, V_REAL, V_PAD, V_PAD, TILES, 1, -100)
    d3 = rlk.make_desc(N, V_REAL, V_PAD, V_PAD, TILES, 3, -100)

    def ws(nbytes):
        return torch.empty(nbytes, dtype=torch.uint8, device=DEV)

    w_fwd = ws(rlk.rlk_logp_workspace_bytes(d1))
    w_one = ws(rlk.rlk_logp_fwd_bwd_workspace_bytes(d3))
    w_ex = ws(rlk.rlk_logp_ex_workspace_bytes(d3))
    w_lm = ws(rlk.rlk_logp_fused_lmhead_workspace_bytes(d3))
    w_onex = ws(rlk.rlk_logp_fwd_bwd_ex_workspace_bytes(d3))
    assert rlk.rlk_logp_fwd_bwd_workspace_bytes(d3) > 256  # both one-launch calls: unit schedule

    def outputs():
        f = lambda: torch.empty(N, device=DEV)  # noqa: E731
        return {"logp": f(), "lse": f(), "d16": torch.empty((N, V_PAD), dtype=torch.bfloat16,
                                                             device=DEV),
                "d32": torch.empty((N, V_PAD), device=DEV), "logp1": f(), "lse1": f(),
                "d1": torch.empty((N, V_PAD), dtype=torch.bfloat16, device=DEV),
                "logpx": f(), "lsex": f(), "ent": f(), "dx": torch.empty((N, V_PAD), device=DEV),
                "lpl": f(), "lsel": f(), "logpy": f(), "lsey": f(), "enty": f(),
                "dy": torch.empty((N, V_PAD), device=DEV)}

    def calls(o):
        x, tg, m, g = st["x"], st["tg"], st["m"], st["g"]
        rlk.rlk_logp_fwd(d1, x, tg, m, o["logp"], o["lse"], w_fwd)
        rlk.rlk_logp_bwd(d1, x, tg, m, o["lse"], g, o["d16"], V_PAD, rlk.RLK_DTYPE_BF16, w_fwd)
        rlk.rlk_logp_bwd(d1, x, tg, m, o["lse"], g, o["d32"], V_PAD, rlk.RLK_DTYPE_F32, w_fwd)
        rlk.rlk_logp_fwd_bwd(d3, x, tg, m, g, o["logp1"], o["lse1"], o["d1"], V_PAD,
                             rlk.RLK_DTYPE_BF16, w_one)
        rlk.rlk_logp_fwd_ex(d3, x, tg, m, o["logpx"], o["lsex"], o["ent"], w_ex)
        rlk.rlk_logp_bwd_ex(d3, x, tg, m, o["lsex"], o["ent"], g, gl, gh, o["dx"], V_PAD,
                            rlk.RLK_DTYPE_F32, w_ex)
        rlk.rlk_logp_fused_lmhead(d3, st["h"], st["w"], K, tg, m, o["lpl"], o["lsel"], w_lm)
        rlk.rlk_logp_fwd_bwd_ex(d3, x, tg, m, g, gl, gh, o["logpy"], o["lsey"], o["enty"],
                                o["dy"], V_PAD, rlk.RLK_DTYPE_F32, w_onex)

    def load(i):
        for k, v in sets[i].items():
            st[k].copy_(v)

    refs = []
    for i in range(len(sets)):  # eager results of every input set
        load(i)
        o = outputs()
        calls(o)
        torch.cuda.synchronize()
        refs.append({k: bits(v) for k, v in o.items()})
    # the one-launch schedule and the separate calls agree, as they must
    for r in refs:
        assert torch.equal(r["logp1"], r["logp"]) and torch.equal(r["d1"], r["d16"])
        assert torch.equal(r["enty"], r["ent"]) and torch.equal(r["dy"], r["dx"])

    og = outputs()
    load(0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(og)
    torch.cuda.synchronize()
    for rep, i in enumerate((1, 0, 2, 2, 1)):
        print(f"replay {rep} on input set {i}", flush=True)
        load(i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in og.items():
            assert torch.equal(bits(v), refs[i][k]), f"{k} differs on replay {rep} (set {i})"
        # eager work between replays, on the same buffers
        rlk.rlk_logp_fwd(d1, st["x"], st["tg"], st["m"], og["logp"], og["lse"], w_fwd)
        torch.cuda.synchronize()
