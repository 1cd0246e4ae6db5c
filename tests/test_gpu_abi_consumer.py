"""The C ABI from plain C: tests/abi_consumer.c links librlk_logp.so and the HIP
runtime only, and checks shard invariance, the exact gather, the backward's row
sums, the one-launch calls against the separate ones bit for bit, and a host
error (see its header).  Needs an MI355X."""
from __future__ import annotations

import subprocess
from pathlib import Path

import pytest

pytestmark = pytest.mark.gpu
BIN = Path(__file__).resolve().parent / "_bin" / "abi_consumer"


def test_plain_c_consumer():
    assert BIN.exists(), "build the C consumer first (__graft_entry__.build())"
    res = subprocess.run([str(BIN)], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all checks passed" in res.stdout
