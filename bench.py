"""Benchmark: one step = forward (per-tile partials + fixed-order merge + gather)
plus backward (dlogits) over the large synthetic workload, on one MI355X.

Prints ONE JSON line on stdout.  Everything else goes to stderr.

  value        algorithmic GB/s of the whole step (logits read twice -- forward
               and backward -- plus the dlogits write and the per-row vectors),
               inputs resident in HBM before the timed region starts
  roofline     the dominant kernel (by time): algorithmic bytes per launch over
               its average launch time, measured with HIP events on the stream
               the kernels run on; traffic = HBM bytes per launch from rocprofv3
               FETCH_SIZE / WRITE_SIZE counters (committed under profiles/),
               reported only while the kernel source is unchanged since then
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same rows
  measured_ceilings
               read-only, write-only and copy stream rates of this GPU from the
               rlk_calib probe (run first, as a child process); roofline then also
               carries frac_of_measured: the time the dominant kernel's reads and
               writes need at those rates, over its measured time
  one_read_accounting
               the same workload counted as one read of every real logit and one
               write of every dX element per step (what the one-launch schedule
               moves), with the two calls' rate under that count and the
               one-launch schedule (rlk_logp_fwd_bwd) timed on the same inputs
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
METRIC = "logits GB/s + tokens/s, fwd+bwd selected-token logp, V=151936; % HBM peak"
KERNEL_SOURCE = ROOT / "vocab_selected_token_amd" / "csrc" / "rlk_kernels.hip"
LMHEAD_SOURCE = ROOT / "vocab_selected_token_amd" / "csrc" / "rlk_lmhead.hip"
TRAFFIC_FILE = ROOT / "profiles" / "traffic_large_32k.txt"
LMHEAD_TRAFFIC_FILE = ROOT / "profiles" / "traffic_lmhead_4096.txt"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(wl, n_active: int) -> dict:
    """Bytes the step must move at minimum (1 GB = 1e9 B).

    forward : every real logit once (2 B) + per row: target 4, mask 1, logp 4, LSE 4
    backward: real logits of effective-active rows (2 B) + every [N, V_pad] dlogit
              written + per row: target 4, mask 1, LSE 4, g 4
    """
    n = wl.num_tokens
    out_b = 2 if wl.dlogits_dtype == "bf16" else 4
    fwd = n * wl.real_vocab * 2 + 13 * n
    bwd = n_active * wl.real_vocab * 2 + n * wl.padded_vocab * out_b + 13 * n
    return {"fwd": fwd, "bwd": bwd}


def algorithmic_bytes_one_pass(wl) -> int:
    """Bytes the one-launch forward+backward must move: every real logit once,
    every [N, V_pad] dlogit written, per row target 4, mask 1, g 4, logp 4, LSE 4."""
    n = wl.num_tokens
    out_b = 2 if wl.dlogits_dtype == "bf16" else 4
    return n * wl.real_vocab * 2 + n * wl.padded_vocab * out_b + 17 * n


def kernel_source_sha(source: Path = KERNEL_SOURCE) -> str:
    """Hash of a kernel source with comments and whitespace removed: it changes
    exactly when the code the counters were taken on changes."""
    text = source.read_text()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


CALIB = Path(__file__).resolve().parent / "vocab_selected_token_amd" / "rlk_calib"


def measured_ceilings():
    """Stream ceilings of this GPU from the rlk_calib probe (8 GiB read-only,
    write-only and copy streams, 16-byte nontemporal accesses, median of 7), run as
    a child process before this one touches the GPU; None if it is not built or
    fails."""
    import subprocess

    if not CALIB.exists():
        return None
    try:
        r = subprocess.run([str(CALIB)], capture_output=True, text=True, timeout=120)
        if r.returncode != 0:
            return None
        out = json.loads(r.stdout.strip().splitlines()[-1])
    except (subprocess.SubprocessError, ValueError, IndexError):
        return None
    out["source"] = ("rlk_calib: 8 GiB streams, 16-byte nontemporal loads/stores, "
                     "1 KB per wave instruction; row_copy and slice_copy copy 32768 rows of "
                     "305,152 bytes one row per block / one sixteenth of a row per block; "
                     "median of 7")
    return out


def read_traffic(kernel: str, workload: str, path: Path = TRAFFIC_FILE,
                 source: Path = KERNEL_SOURCE):
    """HBM bytes per launch of `kernel` from a committed counter summary, or None
    when the summary is missing, was taken on another workload or on a different
    kernel source."""
    if not path.exists():
        return None
    vals = {}
    for line in path.read_text().splitlines():
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if (vals.get("workload") != workload
            or vals.get("kernel_source_sha256") != kernel_source_sha(source)):
        return None
    key = f"{kernel}_hbm_bytes_per_launch"
    return float(vals[key]) if key in vals else None


def unit_fallbacks(ws, kernel: str):
    """Blocks of the last unit-schedule call that computed their row's partials
    themselves instead of receiving them (status word 2 of the workspace); None
    for the row schedule."""
    import torch

    if kernel != "fwd_bwd_units":
        return None
    torch.cuda.synchronize()
    return int(ws[:12].view(torch.int32)[2].item())


def host_cpu() -> dict:
    """The host the oracle runs on: the cores this process may use (its affinity
    mask), the OMP_NUM_THREADS share a shared machine grants one job, the logical
    CPU count, and the model name from /proc/cpuinfo."""
    nproc = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(nproc, int(omp)) if omp.isdigit() and int(omp) > 0 else nproc
    model = "unknown"
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"threads": max(1, threads), "nproc": nproc, "cpu_count": os.cpu_count(),
            "omp_num_threads": omp or None, "cpu_model": model}


def cpu_baseline(inp, wl, max_seconds: float, extended=None, one_pass=False,
                 single_thread_seconds: float = 4.0) -> dict:
    """The oracle (fp64 C, threads over rows) on leading rows of the same workload,
    forward and backward timed separately, on every core the process may use (capped
    by OMP_NUM_THREADS where the machine sets it), plus a single-thread run over the
    first rows.  extended = (g_lse, g_ent) device tensors: time the extended forward
    (entropy) and backward (LSE and entropy gradients) the GPU line runs instead of
    the plain pair.  one_pass: count bytes as the one-launch line does (one read, one
    write)."""
    import numpy as np
    import torch

    import oracle
    import workloads as W

    orc = oracle.get()
    host = host_cpu()
    cores = host["threads"]
    block = 256

    def run(rows, nthreads):
        """(fwd seconds, bwd seconds, fwd bytes, bwd bytes) over one block of rows."""
        bits, tgt, mask, g = W.to_host(inp, rows)
        act = mask & (tgt != W.IGNORE_INDEX)
        if extended is not None:
            sel = torch.as_tensor(rows, device=extended[0].device)
            gl = extended[0][sel].double().cpu().numpy()
            gh = extended[1][sel].double().cpu().numpy()
        t0 = time.perf_counter()
        _, lse, _, _ = orc.fwd(bits, tgt, mask, real_vocab=wl.real_vocab, nthreads=nthreads,
                               raise_on_error=False)
        ent = None
        if extended is not None:
            ent = orc.entropy(bits, real_vocab=wl.real_vocab, nthreads=nthreads)
        t1 = time.perf_counter()
        if extended is None:
            orc.bwd(bits, tgt, mask, lse, g, real_vocab=wl.real_vocab,
                    padded_vocab=wl.padded_vocab, nthreads=nthreads, raise_on_error=False)
        else:
            orc.bwd_ex(bits, tgt, mask, lse, real_vocab=wl.real_vocab,
                       padded_vocab=wl.padded_vocab, ent=ent, g=g, g_lse=gl, g_ent=gh,
                       nthreads=nthreads, raise_on_error=False)
        t2 = time.perf_counter()
        sub = W.Workload(wl.name, 1, len(rows), wl.real_vocab, wl.padded_vocab, wl.sigma,
                         dlogits_dtype=wl.dlogits_dtype)
        b = algorithmic_bytes(sub, int(act.sum()))
        fb, bb = b["fwd"], b["bwd"]
        if one_pass:  # one read of each logit for the whole step: charge it to the forward
            bb = algorithmic_bytes_one_pass(sub) - fb
        if extended is not None:  # as the GPU line counts it
            fb += 4 * len(rows)  # entropy out
            if one_pass:  # grad_lse and grad_ent read; no logit read again
                bb += 8 * len(rows)
            else:  # every row read again, and the entropy read back
                bb += (len(rows) - int(act.sum())) * wl.real_vocab * 2 + 12 * len(rows)
        return t1 - t0, t2 - t1, fb, bb

    def sweep(nthreads, seconds):
        done, tf, tb, bf, bb = 0, 0.0, 0.0, 0, 0
        while done < wl.num_tokens and tf + tb < seconds:
            rows = np.arange(done, min(wl.num_tokens, done + block))
            a, b, c, d = run(rows, nthreads)
            tf, tb, bf, bb = tf + a, tb + b, bf + c, bb + d
            done += len(rows)
        return done, tf, tb, bf, bb

    done, tf, tb, bf, bb = sweep(cores, max_seconds)
    done1, tf1, tb1, bf1, bb1 = sweep(1, single_thread_seconds)
    what = ("fwd with entropy + bwd with LSE and entropy gradients" if extended is not None
            else "fwd+bwd")
    rate = lambda nbytes, sec: round(nbytes / sec / 1e9, 4)
    return {"value": rate(bf + bb, tf + tb), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"rows 0..{done - 1} of the same workload ({done} of {wl.num_tokens} "
                      f"rows), {what} in fp64 on {cores} threads, {tf + tb:.1f} s; the single-"
                      f"thread run took rows 0..{done1 - 1}",
            "tokens_per_s": round(done / (tf + tb), 2),
            "fwd": {"GB/s": rate(bf, tf), "tokens_per_s": round(done / tf, 2),
                    "seconds": round(tf, 3)},
            "bwd": {"GB/s": rate(bb, tb), "tokens_per_s": round(done / tb, 2),
                    "seconds": round(tb, 3)},
            "single_thread": {"GB/s": rate(bf1 + bb1, tf1 + tb1), "rows": done1,
                              "fwd_GB/s": rate(bf1, tf1), "bwd_GB/s": rate(bb1, tb1),
                              "tokens_per_s": round(done1 / (tf1 + tb1), 2)},
            "host": host}


def sha256_device(t, chunk_bytes: int = 1 << 28) -> str:
    """SHA-256 of a device tensor's bytes, copied to the host in chunks."""
    import torch

    flat = t.detach().contiguous().view(-1).view(torch.uint8)
    h = hashlib.sha256()
    for o in range(0, flat.numel(), chunk_bytes):
        h.update(flat[o:o + chunk_bytes].cpu().numpy().tobytes())
    return h.hexdigest()


def fingerprints(rlk, wl, inp, mask_u8, shard_counts=(1, 8)) -> dict:
    """SHA-256 of one batch's inputs, and of the fp32 logp and LSE the forward gives
    for it at each virtual-shard count (the cross-grouping bitwise check): the digests
    must agree for every count."""
    import torch

    import workloads as W

    n = wl.num_tokens
    dev = inp.logits.device
    out = {"inputs": {"logits": sha256_device(inp.logits), "targets": sha256_device(inp.targets),
                      "mask": sha256_device(mask_u8), "grad": sha256_device(inp.grad)}}
    per = {}
    for s in shard_counts:
        desc = rlk.make_desc(n, wl.real_vocab, wl.padded_vocab, wl.ld_logits, wl.num_tiles, s,
                             W.IGNORE_INDEX)
        ws = rlk.workspace_for(desc, dev)
        logp = torch.empty(n, dtype=torch.float32, device=dev)
        lse = torch.empty(n, dtype=torch.float32, device=dev)
        rlk.rlk_logp_fwd(desc, inp.logits, inp.targets, mask_u8, logp, lse, ws,
                         torch.cuda.current_stream())
        torch.cuda.synchronize()
        per[str(s)] = {"logp": sha256_device(logp), "lse": sha256_device(lse)}
        del ws
    out["outputs_by_virtual_shards"] = per
    out["outputs_identical_across_shards"] = len({(v["logp"], v["lse"]) for v in per.values()}) == 1
    return out


def copy_probe(args, dev) -> None:
    """A plain copy of known size (untimed), whose FETCH_SIZE / WRITE_SIZE readings
    scale the counters of the kernels in the same profiled run."""
    import torch

    if args.copy_probe_gib <= 0:
        return
    nbytes = int(args.copy_probe_gib * 2 ** 30)
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"bench: copy probe {nbytes} bytes x3 done")
    del src, dst


LMHEAD_WORKLOAD = "lmhead_b4096_k4096_v151936_p152576"
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, vendor figure


def cpu_baseline_lmhead(h, w, tgt, v_real: int, max_seconds: float) -> dict:
    """The oracle (z = h . W^T in fp64 with plain loops, threads over vocabulary columns,
    then the fp64 log-softmax) on leading tokens of the LM-head workload."""
    import numpy as np
    import torch

    import oracle

    orc = oracle.get()
    host = host_cpu()
    cores = host["threads"]
    n, k = h.shape
    hb = h.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    wb = w[:v_real].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    tg = tgt.cpu().numpy()
    block = 4
    done, elapsed = 0, 0.0
    while done < n and elapsed < max_seconds:
        r1 = min(n, done + block)
        t0 = time.perf_counter()
        z = orc.lmhead_logits(hb[done:r1], wb, real_vocab=v_real, nthreads=cores)
        orc.fwd(z, tg[done:r1], None, real_vocab=v_real, nthreads=cores, raise_on_error=False)
        elapsed += time.perf_counter() - t0
        done = r1
    flops = 2.0 * done * v_real * k
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"tokens 0..{done - 1} of the same workload ({done} of {n} tokens): "
                      f"h . W^T in fp64, then the fp64 log-softmax, {elapsed:.1f} s",
            "tokens_per_s": round(done / elapsed, 3), "host": host}


def bench_lmhead(args) -> int:
    """The fused LM-head variant: hidden [4096, 4096] ~ N(0,1), W [152576, 4096] ~ N(0, 0.02^2),
    rows >= 151936 padding, 64 tiles, all tokens active, forward only."""
    import torch

    import vocab_selected_token_amd as rlk

    dev = torch.device("cuda", 0)
    n, k, v_real, v_pad, tiles = 4096, 4096, 151936, 152576, 64
    g = torch.Generator(device=dev).manual_seed(123)
    h = torch.randn((n, k), generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn((v_pad, k), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    tgt = torch.randint(0, v_real, (n,), generator=g, device=dev, dtype=torch.int32)
    desc = rlk.make_desc(n, v_real, v_pad, v_pad, tiles, args.shards, -100)
    ws = torch.empty(rlk.rlk_logp_fused_lmhead_workspace_bytes(desc), dtype=torch.uint8,
                     device=dev)
    logp = torch.empty(n, device=dev)
    lse = torch.empty(n, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        rlk.rlk_logp_fused_lmhead(desc, h, w, k, tgt, None, logp, lse, ws, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        rlk.rlk_logp_fused_lmhead(desc, h, w, k, tgt, None, logp, lse, ws, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    flops = 2.0 * n * v_real * k  # padding rows are not computed
    tflops = flops / (ev_ms * 1e-3) / 1e12
    library = None
    if args.library_gemm:  # context only: the plain library GEMM h . W^T of the same shape
        wr = w[:v_real]
        for _ in range(2):
            torch.matmul(h, wr.t())
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            torch.matmul(h, wr.t())
        e1.record(stream)
        torch.cuda.synchronize()
        lib_ms = e0.elapsed_time(e1) / args.steps
        library = {"ms": round(lib_ms, 4), "TFLOP/s": round(flops / (lib_ms * 1e-3) / 1e12, 1),
                   "note": "torch.matmul bf16 -> bf16 logits (materialised), no logp"}
    copy_probe(args, dev)
    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline_lmhead(h, w, tgt, v_real, args.cpu_seconds)
    line = {
        "metric": "fused LM-head selected-token logp, TFLOP/s (MFMA utilisation)",
        "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": LMHEAD_WORKLOAD, "tokens": n, "hidden": k, "real_vocab": v_real,
                   "padded_vocab": v_pad, "vocab_tiles": tiles,
                   "virtual_shards": args.shards},
        "tokens_per_s": round(n / (ev_ms * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": read_traffic("lmhead_segments", LMHEAD_WORKLOAD, LMHEAD_TRAFFIC_FILE,
                                             LMHEAD_SOURCE),
                     "kernel": "lmhead_segments+lmhead_tiles+stage2_merge"},
        "cpu_baseline": cpu,
        "library_gemm": library,
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fwd_bwd_b8s4096_v151936_p152576")
    ap.add_argument("--shards", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-alt-schedule", action="store_true",
                    help="skip timing the one-launch schedule beside the two calls")
    ap.add_argument("--one-pass", action="store_true",
                    help="time rlk_logp_fwd_bwd (g known before the forward) instead of "
                         "rlk_logp_fwd + rlk_logp_bwd")
    ap.add_argument("--extended", action="store_true",
                    help="time rlk_logp_fwd_ex + rlk_logp_bwd_ex (entropy output; logp, LSE "
                         "and entropy gradients) instead of rlk_logp_fwd + rlk_logp_bwd; with "
                         "--one-pass, rlk_logp_fwd_bwd_ex")
    ap.add_argument("--library-gemm", action="store_true",
                    help="LM-head workload: also time the library GEMM of the same shape")
    ap.add_argument("--no-sha", action="store_true",
                    help="skip the SHA-256 fingerprints of the inputs and of logp/LSE at S = 1, 8")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the stream-ceiling probe reported beside the roofline")
    ap.add_argument("--copy-probe-gib", type=float, default=0.0,
                    help="also run an untimed plain copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path is single-device by design", file=sys.stderr)
        return 2

    ceilings = None
    if not args.no_ceilings and args.workload != LMHEAD_WORKLOAD:
        log("bench: measuring stream ceilings (rlk_calib)")
        ceilings = measured_ceilings()

    if args.workload == LMHEAD_WORKLOAD:
        return bench_lmhead(args)

    import torch

    import workloads as W
    import vocab_selected_token_amd as rlk

    wl = W.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"bench: workload {wl.name}, generating inputs on {torch.cuda.get_device_name(dev)}")
    # Two independent batches, used alternately, so that no step reads logits
    # another step left in the GPU's caches.
    inps = [W.make_inputs(wl, dev), W.make_inputs(wl, dev, seed=wl.seed + 1)]
    inp = inps[0]
    n = wl.num_tokens
    act = inp.mask & (inp.targets != W.IGNORE_INDEX)
    n_active = int(act.sum())
    act1 = inps[1].mask & (inps[1].targets != W.IGNORE_INDEX)
    # algorithmic bytes averaged over the two batches (they differ in active rows only)
    nb0, nb1 = algorithmic_bytes(wl, n_active), algorithmic_bytes(wl, int(act1.sum()))
    nb = {k: (nb0[k] + nb1[k]) // 2 for k in nb0}

    desc = rlk.make_desc(n, wl.real_vocab, wl.padded_vocab, wl.ld_logits, wl.num_tiles,
                         args.shards, W.IGNORE_INDEX)
    # one workspace for every schedule timed here: the separate calls' partials, or
    # the one-launch schedule's partial slots
    ws = torch.empty(max(rlk.rlk_logp_workspace_bytes(desc),
                         rlk.rlk_logp_fwd_bwd_workspace_bytes(desc)), dtype=torch.uint8,
                     device=dev)
    one_kernel = ("fwd_bwd_units" if rlk.rlk_logp_fwd_bwd_workspace_bytes(desc) > 256
                  else "fwd_bwd_rows")
    logp = torch.empty(n, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    out_dt = torch.bfloat16 if wl.dlogits_dtype == "bf16" else torch.float32
    ld_d = (wl.padded_vocab + 7) // 8 * 8
    dl = torch.empty((n, ld_d), dtype=out_dt, device=dev) if wl.backward else None
    code = rlk.RLK_DTYPE_BF16 if out_dt == torch.bfloat16 else rlk.RLK_DTYPE_F32
    masks = [b.mask.view(torch.uint8) for b in inps]
    stream = torch.cuda.current_stream()

    one_pass = args.one_pass
    extended = args.extended
    if (one_pass or extended) and not wl.backward:
        log("bench: --one-pass and --extended need a forward+backward workload")
        return 2
    if extended:
        ws = torch.empty(max(rlk.rlk_logp_ex_workspace_bytes(desc),
                             rlk.rlk_logp_fwd_bwd_ex_workspace_bytes(desc) if one_pass else 0),
                         dtype=torch.uint8, device=dev)
        ent = torch.empty(n, dtype=torch.float32, device=dev)
        gx = torch.Generator(device=dev).manual_seed(wl.seed + 7)
        g_lse = torch.randn(n, generator=gx, device=dev)
        g_ent = torch.randn(n, generator=gx, device=dev)

    def step(i, events=None):
        b, m = inps[i % 2], masks[i % 2]
        if events:
            events[0].record(stream)
        if one_pass and extended:
            rlk.rlk_logp_fwd_bwd_ex(desc, b.logits, b.targets, m, b.grad, g_lse, g_ent, logp, lse,
                                    ent, dl, ld_d, code, ws, stream)
            if events:
                events[1].record(stream)
                events[2].record(stream)
            return
        if one_pass:
            rlk.rlk_logp_fwd_bwd(desc, b.logits, b.targets, m, b.grad, logp, lse, dl, ld_d, code,
                                 ws, stream)
            if events:
                events[1].record(stream)
                events[2].record(stream)
            return
        if extended:
            rlk.rlk_logp_fwd_ex(desc, b.logits, b.targets, m, logp, lse, ent, ws, stream)
        else:
            rlk.rlk_logp_fwd(desc, b.logits, b.targets, m, logp, lse, ws, stream)
        if events:
            events[1].record(stream)
        if extended:
            rlk.rlk_logp_bwd_ex(desc, b.logits, b.targets, m, lse, ent, b.grad, g_lse, g_ent, dl,
                                ld_d, code, ws, stream)
        elif wl.backward:
            rlk.rlk_logp_bwd(desc, b.logits, b.targets, m, lse, b.grad, dl, ld_d, code, ws, stream)
        if events:
            events[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps if wl.backward else 0.0
    # spread of the individual steps as the stream saw them (events around each step)
    per_step = sorted(e[0].elapsed_time(e[2]) for e in evs)
    pick = lambda q: per_step[min(len(per_step) - 1, int(q * (len(per_step) - 1) + 0.5))]
    step_spread = {"p10": round(pick(0.1), 4), "p50": round(pick(0.5), 4),
                   "p90": round(pick(0.9), 4)}
    log(f"bench: {ms_step:.3f} ms/step (fwd {fwd_ms:.3f} ms, bwd {bwd_ms:.3f} ms; "
        f"step p10/p50/p90 {step_spread['p10']}/{step_spread['p50']}/{step_spread['p90']} ms)")

    # The same workload under the other accounting: one read of every real logit and
    # one write of every dX element per step, which only the one-launch schedule
    # (rlk_logp_fwd_bwd, for a g known before the forward) reaches; timed on the
    # same inputs so that both schedules appear in the one line.
    one_read = None
    if wl.backward and not one_pass and not extended and not args.no_alt_schedule:
        def step_one(i):
            b, m = inps[i % 2], masks[i % 2]
            rlk.rlk_logp_fwd_bwd(desc, b.logits, b.targets, m, b.grad, logp, lse, dl, ld_d, code,
                                 ws, stream)
        for i in range(args.warmup):
            step_one(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step_one(i)
        torch.cuda.synchronize()
        ms_one = (time.perf_counter() - t0) * 1e3 / args.steps
        fallbacks = unit_fallbacks(ws, one_kernel)
        b_one = algorithmic_bytes_one_pass(wl)
        one_read = {"bytes_per_step": b_one,
                    "two_calls_GB/s": round(b_one / (ms_step * 1e-3) / 1e9, 1),
                    "two_calls_hbm_frac": round(b_one / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "one_launch_ms_per_step": round(ms_one, 4),
                    "one_launch_GB/s": round(b_one / (ms_one * 1e-3) / 1e9, 1),
                    "one_launch_hbm_frac": round(b_one / (ms_one * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "one_launch_tokens_per_s": round(n / (ms_one * 1e-3), 1),
                    "one_launch_kernel": one_kernel,
                    "one_launch_fallback_blocks": fallbacks}
        if ceilings is not None and "row_copy_GBps" in ceilings:
            # what a copy of the same bytes takes on this GPU in the two shapes such a
            # schedule can have, with no arithmetic at all (rlk_calib)
            one_read["row_copy_ms"] = round(b_one / (ceilings["row_copy_GBps"] * 1e9) * 1e3, 4)
            one_read["slice_copy_ms"] = round(b_one / (ceilings["slice_copy_GBps"] * 1e9) * 1e3,
                                              4)
            one_read["one_launch_frac_of_row_copy"] = round(one_read["row_copy_ms"] / ms_one, 4)
            one_read["slice_copy_hbm_frac"] = round(ceilings["slice_copy_GBps"] / HBM_PEAK_GBS,
                                                    4)
        log(f"bench: one-launch schedule {ms_one:.3f} ms/step")

    copy_probe(args, dev)

    shas = None
    if not args.no_sha:
        log("bench: SHA-256 of the inputs and of logp/LSE at S = 1 and 8")
        shas = fingerprints(rlk, wl, inps[0], masks[0])

    if one_pass:
        # with the extended form: the entropy written, grad_lse and grad_ent read
        total_bytes = algorithmic_bytes_one_pass(wl) + (12 * n if extended else 0)
        value = total_bytes / (ms_step * 1e-3) / 1e9
        k_gbs = total_bytes / (fwd_ms * 1e-3) / 1e9
        kname = one_kernel + ("_ex" if extended else "")
        kernels = {kname: {"ms": round(fwd_ms, 4), "GB/s": round(k_gbs, 1),
                           "bytes": total_bytes,
                           "fallback_blocks": unit_fallbacks(ws, one_kernel)}}
        roofline = {"bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                    "traffic": None if extended else read_traffic(one_kernel, wl.name),
                    "kernel": kname}
    else:
        if extended:  # every row's logits are read again (the LSE and entropy terms reach all)
            nb = dict(nb)
            nb["fwd"] += 4 * n  # entropy out
            nb["bwd"] += (n - (n_active + int(act1.sum())) // 2) * wl.real_vocab * 2 + 12 * n
        total_bytes = nb["fwd"] + (nb["bwd"] if wl.backward else 0)
        value = total_bytes / (ms_step * 1e-3) / 1e9
        fwd_gbs = nb["fwd"] / (fwd_ms * 1e-3) / 1e9
        kernels = {"stage1_partials+stage2_merge": {"ms": round(fwd_ms, 4),
                                                    "GB/s": round(fwd_gbs, 1),
                                                    "bytes": nb["fwd"]}}
        if wl.backward:
            bwd_gbs = nb["bwd"] / (bwd_ms * 1e-3) / 1e9
            kernels["bwd_dlogits"] = {"ms": round(bwd_ms, 4), "GB/s": round(bwd_gbs, 1),
                                      "bytes": nb["bwd"]}
        dom = ("bwd_dlogits" if wl.backward and bwd_ms >= fwd_ms
               else "stage1_partials+stage2_merge")
        dom_gbs = kernels[dom]["GB/s"]
        roofline = {"bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                    "traffic": None if extended else read_traffic(
                        "bwd_dlogits" if dom == "bwd_dlogits" else "stage1", wl.name),
                    "kernel": dom}

    # the dominant kernel against this GPU's measured stream ceilings: the time its
    # reads need at the read-only rate plus the time its dX writes need at the
    # write-only rate, over its measured time
    if ceilings is not None:
        out_b = 2 if wl.dlogits_dtype == "bf16" else 4
        k_ms = fwd_ms if (one_pass or roofline["kernel"] != "bwd_dlogits") else bwd_ms
        k_bytes = kernels[roofline["kernel"]]["bytes"]
        k_write = n * wl.padded_vocab * out_b if (one_pass or wl.backward and
                                                  roofline["kernel"] == "bwd_dlogits") else 0
        bound_ms = ((k_bytes - k_write) / (ceilings["read_GBps"] * 1e9)
                    + k_write / (ceilings["write_GBps"] * 1e9)) * 1e3
        roofline["frac_of_measured"] = round(bound_ms / k_ms, 4)
        roofline["measured_bound_ms"] = round(bound_ms, 4)

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(inp, wl, args.cpu_seconds,
                           extended=(g_lse, g_ent) if extended else None, one_pass=one_pass)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "input_dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": n, "active_tokens": n_active,
                   "real_vocab": wl.real_vocab, "padded_vocab": wl.padded_vocab,
                   "vocab_tiles": wl.num_tiles, "virtual_shards": args.shards,
                   "dlogits_dtype": wl.dlogits_dtype, "parallelism": "single-gpu",
                   "schedule": ("one launch (rlk_logp_fwd_bwd_ex: entropy; logp, LSE and "
                                "entropy gradients)" if one_pass and extended
                                else "one launch (rlk_logp_fwd_bwd)" if one_pass
                                else "rlk_logp_fwd_ex then rlk_logp_bwd_ex (entropy; logp, LSE "
                                "and entropy gradients)" if extended
                                else "rlk_logp_fwd then rlk_logp_bwd")},
        "tokens_per_s": round(n / (ms_step * 1e-3), 1),
        "step_ms_stream": step_spread,
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        # the same step counted the way the workload's own description counts it:
        # one read of every real logit and one write of every dX element
        "hbm_frac_one_read": (round(algorithmic_bytes_one_pass(wl) / (ms_step * 1e-3) / 1e9
                                    / HBM_PEAK_GBS, 4) if wl.backward and not extended
                              else None),
        "algorithmic_bytes_per_step": total_bytes,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if one_read is not None:
        line["one_read_accounting"] = one_read
    line["measured_ceilings"] = ceilings
    line["sha256"] = shas
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
