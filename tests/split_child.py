"""Child process of the split-launch GPU test: runs every entry point on one fixed,
seeded case and saves the output bits to the path it is given.  The library reads
RLK_MAX_LAUNCH_THREADS once per process, so the test starts this module once per
launch limit with the variable set in its environment.

    python -m tests.split_child OUT.pt
"""
from __future__ import annotations

import sys

import torch

import vocab_selected_token_amd as rlk
import workloads as W

DEV = torch.device("cuda")


def bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def make_case():
    """300 rows of 5120 columns (5000 real), 64 tiles; and a 300-token LM-head case
    with K = 128 over 5120 weight rows (5000 real), 16 tiles."""
    wl = W.small_workload(300, 5000, 5120, num_tiles=64, sigma=2.0, mask_keep=0.8,
                          ignore_frac=0.05, seed=77)
    inp = W.make_inputs(wl, DEV)
    gen = torch.Generator(device="cpu").manual_seed(78)
    n_tok, k, v_real, v_pad, t = 300, 128, 5000, 5120, 16
    h = (torch.randn(n_tok, k, generator=gen)).to(torch.bfloat16).to(DEV)
    w = (torch.randn(v_pad, k, generator=gen) * 0.1).to(torch.bfloat16).to(DEV)
    tg = torch.randint(0, v_real, (n_tok,), generator=gen, dtype=torch.int32).to(DEV)
    return inp, wl, (h, w, tg, v_real, v_pad, t)


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
    # the unit schedule's fallback counter (status word 2) after a bf16 call
    d = rlk.make_desc(wl.num_tokens, wl.real_vocab, wl.padded_vocab, wl.ld_logits, wl.num_tiles)
    ws = torch.empty(rlk.rlk_logp_fwd_bwd_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    rlk.forward_backward(inp.logits, inp.targets, inp.mask, inp.grad, out_dtype=torch.bfloat16,
                         workspace=ws, **kw)
    torch.cuda.synchronize()
    out["one_fallbacks"] = (ws[:12].view(torch.int32)[2:3].clone(),)
    gl = torch.linspace(-1.0, 1.0, wl.num_tokens, device=DEV)
    out["bwd_ex"] = (rlk.backward_ex(inp.logits, inp.targets, inp.mask, lse, ent, inp.grad, gl,
                                     -gl, **kw),)
    # the extended one launch, and its fallback counter
    wse = torch.empty(rlk.rlk_logp_fwd_bwd_ex_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    out["one_ex"] = rlk.forward_backward_ex(inp.logits, inp.targets, inp.mask, inp.grad, gl, -gl,
                                            out_dtype=torch.bfloat16, workspace=wse, **kw)
    torch.cuda.synchronize()
    out["one_ex_fallbacks"] = (wse[:12].view(torch.int32)[2:3].clone(),)
    h, w, tg, v_real, v_pad, t = lm
    out["lmhead"] = rlk.fused_lmhead(h, w, tg, real_vocab=v_real, padded_vocab=v_pad,
                                     num_vocab_tiles=t)
    out["lmhead_s3"] = rlk.fused_lmhead(h, w, tg, real_vocab=v_real, padded_vocab=v_pad,
                                        num_vocab_tiles=t, num_virtual_shards=3)
    torch.cuda.synchronize()
    return {k: tuple(bits(x).cpu() for x in v) for k, v in out.items()}


def main(out_path: str) -> int:
    print("split child: running every entry point", flush=True)
    res = run_all(*make_case())
    torch.save(res, out_path)
    print("split child: done", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
