"""Seeded synthetic workloads for selected-token logp (input synthesis only).

This module holds no part of the method's arithmetic: it draws logits,
targets, masks and upstream gradients with one torch generator and serves the
same tensors to the GPU path and (after a host copy) to the CPU oracle.

Shapes come from the pages: Issue #323 "H100 validation and reproduction guide
for Issue #241 PR1-PR5", "2. Six-Case TP/CP Matrix" (batch 2, sequence 16,
8 prompt tokens, real = padded vocabulary 151936, 64 tiles, seed 123), and the
H100 canonical TP/CP validation page, "Fixes exercised" (vocabulary padded to
152576, 1024-token microbatches).  The value distributions, masks and larger
batches are this library's benchmark recipe.

Recipe for one workload (all draws from ``torch.Generator(device).manual_seed(seed)``,
in this order):
  1. targets  ~ U{0, ..., V_real - 1}, int32 [N]
  2. mask     ~ Bernoulli(mask_keep) [N] if mask_keep is set, else all True;
                then positions < prompt_inactive of every sequence are set False
  3. spike    rows ~ Bernoulli(spike_frac) [N] (drawn only if spike_frac > 0)
  4. ignore   rows ~ Bernoulli(ignore_frac) [N] (drawn only if ignore_frac > 0);
                their targets become ignore_index (after the spike was placed)
  5. g        ~ N(0, 1) fp32 [N]
  6. logits   rows in chunks of 1024: fp32 N(0, sigma^2) over [0, V_real), plus
                `spike` at the target column of spike rows, rounded to bf16 (RNE)
  7. padding  columns [V_real, ld) hold uniform random 16-bit patterns (NaN and
                Inf encodings included): the path must never let them count
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np
import torch

IGNORE_INDEX = -100
GEN_CHUNK_ROWS = 1024


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq: int
    real_vocab: int
    padded_vocab: int
    sigma: float
    num_tiles: int = 64
    prompt_inactive: int = 0
    mask_keep: float | None = None
    spike_frac: float = 0.0
    spike: float = 0.0
    ignore_frac: float = 0.0
    backward: bool = True
    dlogits_dtype: str = "f32"  # "f32" or "bf16"
    shards: tuple = (1,)
    ld: int | None = None  # defaults to padded_vocab rounded up to 8
    seed: int = 123
    note: str = field(default="", compare=False)

    @property
    def num_tokens(self) -> int:
        return self.batch * self.seq

    @property
    def ld_logits(self) -> int:
        return self.ld if self.ld is not None else (self.padded_vocab + 7) // 8 * 8


MATRIX_B2S16 = Workload(
    "matrix_b2s16_v151936", batch=2, seq=16, real_vocab=151936, padded_vocab=151936, sigma=2.0,
    prompt_inactive=8, backward=True, dlogits_dtype="f32", shards=(1, 2, 4, 8),
    note="the pages' six-case matrix shape; fwd+bwd, fp32 dlogits")
MICROBATCH_1024 = Workload(
    "microbatch_b8s128_v151936_p152576", batch=8, seq=128, real_vocab=151936,
    padded_vocab=152576, sigma=3.0, mask_keep=0.75, spike_frac=0.2, spike=12.0,
    ignore_frac=0.03, backward=True, dlogits_dtype="f32",
    note="1024-token microbatch, padded vocabulary with garbage padding; fwd+bwd")
THROUGHPUT_16K = Workload(
    "fwd_b16s1024_v151936", batch=16, seq=1024, real_vocab=151936, padded_vocab=151936,
    sigma=2.0, backward=False, shards=(1, 2, 4, 8),
    note="forward only, run at 1/2/4/8 virtual shards; SHA-256 must match")
LARGE_32K = Workload(
    "fwd_bwd_b8s4096_v151936_p152576", batch=8, seq=4096, real_vocab=151936,
    padded_vocab=152576, sigma=2.5, prompt_inactive=512, ignore_frac=0.05, backward=True,
    dlogits_dtype="bf16", note="large fwd+bwd, bf16 dlogits (~10 GB logits + ~10 GB dlogits)")

WORKLOADS = {w.name: w for w in (MATRIX_B2S16, MICROBATCH_1024, THROUGHPUT_16K, LARGE_32K)}


@dataclass
class Inputs:
    wl: Workload
    logits: torch.Tensor  # bf16 [N, ld]
    targets: torch.Tensor  # int32 [N]
    mask: torch.Tensor  # bool [N]
    grad: torch.Tensor  # fp32 [N]


def make_inputs(wl: Workload, device="cpu", seed: int | None = None) -> Inputs:
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed if seed is None else seed)
    n, v_real, ld = wl.num_tokens, wl.real_vocab, wl.ld_logits
    targets = torch.randint(0, v_real, (n,), generator=gen, device=device,
                            dtype=torch.int64).to(torch.int32)
    if wl.mask_keep is not None:
        mask = torch.rand(n, generator=gen, device=device) < wl.mask_keep
    else:
        mask = torch.ones(n, dtype=torch.bool, device=device)
    if wl.prompt_inactive:
        pos = torch.arange(n, device=device) % wl.seq
        mask &= pos >= wl.prompt_inactive
    spike_rows = None
    if wl.spike_frac > 0:
        spike_rows = torch.rand(n, generator=gen, device=device) < wl.spike_frac
    spike_cols = targets.clone()
    if wl.ignore_frac > 0:
        ign = torch.rand(n, generator=gen, device=device) < wl.ignore_frac
        targets[ign] = IGNORE_INDEX
    grad = torch.randn(n, generator=gen, device=device, dtype=torch.float32)

    logits = torch.empty((n, ld), dtype=torch.bfloat16, device=device)
    for r0 in range(0, n, GEN_CHUNK_ROWS):
        r1 = min(n, r0 + GEN_CHUNK_ROWS)
        x = torch.randn((r1 - r0, v_real), generator=gen, device=device, dtype=torch.float32)
        x.mul_(wl.sigma)
        if spike_rows is not None:
            rows = torch.nonzero(spike_rows[r0:r1]).flatten()
            x[rows, spike_cols[r0:r1][rows].long()] += wl.spike
        logits[r0:r1, :v_real] = x.to(torch.bfloat16)
        del x
    if ld > v_real:
        pad = torch.randint(-32768, 32768, (n, ld - v_real), generator=gen, device=device,
                            dtype=torch.int32).to(torch.int16)
        logits[:, v_real:] = pad.view(torch.bfloat16)
        del pad
    return Inputs(wl, logits, targets, mask, grad)


def small_workload(n: int, real_vocab: int, padded_vocab: int | None = None, *,
                   ld: int | None = None, num_tiles: int = 64, sigma: float = 2.0,
                   mask_keep: float | None = 0.8, ignore_frac: float = 0.1,
                   spike_frac: float = 0.0, spike: float = 0.0, seed: int = 7,
                   dlogits_dtype: str = "f32") -> Workload:
    """An ad-hoc workload for parity tests (one sequence of n tokens)."""
    return Workload(f"small_n{n}_v{real_vocab}", batch=1, seq=n, real_vocab=real_vocab,
                    padded_vocab=padded_vocab or real_vocab, sigma=sigma, num_tiles=num_tiles,
                    mask_keep=mask_keep, ignore_frac=ignore_frac, spike_frac=spike_frac,
                    spike=spike, dlogits_dtype=dlogits_dtype, ld=ld, seed=seed)


def to_host(inp: Inputs, rows=None):
    """numpy copies for the oracle: (logits bf16 bits uint16, targets, mask, grad float64)."""
    sel = slice(None) if rows is None else torch.as_tensor(rows, device=inp.logits.device)
    bits = inp.logits[sel].view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits, inp.targets[sel].cpu().numpy(), inp.mask[sel].cpu().numpy(),
            inp.grad[sel].double().cpu().numpy())


def sha256(t: torch.Tensor) -> str:
    return hashlib.sha256(t.detach().contiguous().cpu().view(torch.uint8).numpy().tobytes()
                          ).hexdigest()
