"""The benchmark's contract on the CPU: the one-GPU guard, and the byte counts its
rates are computed from, against sums written out by hand for the 32768-row
workload (32768 x 152576 columns, 151936 real, bf16 dX)."""
from __future__ import annotations

import subprocess
import sys
from pathlib import Path

import bench
import workloads as W

ROOT = Path(__file__).resolve().parent.parent


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert r.stdout == ""  # no JSON line
    assert "one GPU" in r.stderr


def test_byte_counts_of_the_large_workload():
    wl = W.LARGE_32K
    n, real, pad = 32768, 151936, 152576
    assert (wl.num_tokens, wl.real_vocab, wl.padded_vocab, wl.dlogits_dtype) == \
        (n, real, pad, "bf16")
    active = 27193
    b = bench.algorithmic_bytes(wl, active)
    # forward: each real logit once (bf16), and per row target 4 + mask 1 + logp 4 + LSE 4
    assert b["fwd"] == n * real * 2 + n * (4 + 1 + 4 + 4) == 9_957_703_680
    # backward: the active rows' real logits, every bf16 dX element, and per row
    # target 4 + mask 1 + LSE 4 + g 4
    assert b["bwd"] == active * real * 2 + n * pad * 2 + n * 13
    # one launch: each real logit read once, each dX element written once, and per
    # row target 4 + mask 1 + g 4 + logp 4 + LSE 4
    assert bench.algorithmic_bytes_one_pass(wl) == n * real * 2 + n * pad * 2 + 17 * n \
        == 19_957_055_488


def test_fp32_dlogits_count_four_bytes():
    wl = W.MICROBATCH_1024
    assert wl.dlogits_dtype == "f32"
    b = bench.algorithmic_bytes(wl, 0)
    assert b["bwd"] == wl.num_tokens * wl.padded_vocab * 4 + 13 * wl.num_tokens


def test_committed_traffic_matches_the_current_kernels():
    """The counter summaries under profiles/ were taken on the kernel sources as they
    stand (the bench line reports traffic only while the hashes agree)."""
    big = W.LARGE_32K.name
    assert bench.read_traffic("bwd_dlogits", big) is not None
    assert bench.read_traffic("stage1", big) is not None
    assert bench.read_traffic("fwd_bwd_units", big) is not None
    assert bench.read_traffic("lmhead_segments", bench.LMHEAD_WORKLOAD, bench.LMHEAD_TRAFFIC_FILE,
                              bench.LMHEAD_SOURCE) is not None


def test_traffic_is_reported_only_for_the_workload_it_was_taken_on():
    """The counters were taken on the 32768-row and the 4096-token LM-head workloads;
    a bench line for any other workload carries no traffic figure."""
    for wl in (W.MATRIX_B2S16, W.MICROBATCH_1024, W.THROUGHPUT_16K):
        for k in ("bwd_dlogits", "stage1", "fwd_bwd_units"):
            assert bench.read_traffic(k, wl.name) is None
    assert bench.read_traffic("lmhead_segments", W.LARGE_32K.name,
                              bench.LMHEAD_TRAFFIC_FILE, bench.LMHEAD_SOURCE) is None


def test_no_undefined_global_names():
    """Every global name a function of the bench, the input generators, the entry
    points or the binding reads exists in its module or in builtins (the GPU-only
    code paths of these files do not run on the CPU)."""
    import builtins
    import importlib
    import symtable

    for name in ("bench", "workloads", "__graft_entry__", "vocab_selected_token_amd"):
        mod = importlib.import_module(name)
        src = Path(mod.__file__).read_text()
        missing = []

        def walk(t):
            for s in t.get_symbols():
                n = s.get_name()
                if (s.is_referenced() and s.is_global() and not hasattr(mod, n)
                        and not hasattr(builtins, n)):
                    missing.append((t.get_name(), n))
            for c in t.get_children():
                walk(c)

        walk(symtable.symtable(src, mod.__file__, "exec"))
        assert missing == [], (name, missing)
