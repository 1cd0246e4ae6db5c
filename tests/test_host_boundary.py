"""Host-side checks of the C-ABI library (no GPU: nothing here launches a kernel).

* the library loads and exports every function include/rlk_logp.h declares;
* descriptor / pointer / size validation returns the documented status codes
  before anything is enqueued;
* the host geometry helper agrees with the oracle's geometry and with the
  pages' sizes (64 tiles of 2374 columns over 151936, of 2384 over 152576).
"""
from __future__ import annotations

import ctypes
import re
import subprocess
from pathlib import Path

import numpy as np
import pytest

import oracle
import vocab_selected_token_amd as rlk

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "rlk_logp.h"


def declared_functions() -> set[str]:
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(rlk_[a-z0-9_]+)\s*\(", text))


def test_header_declares_the_boundary():
    assert declared_functions() == set(rlk.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(str(rlk.LIB_PATH))
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", str(rlk.LIB_PATH)], check=True,
                         capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert declared_functions() <= exported


def test_library_does_not_link_the_oracle():
    out = subprocess.run(["nm", "-D", str(rlk.LIB_PATH)], check=True, capture_output=True,
                         text=True).stdout
    assert "rlk_oracle" not in out
    deps = subprocess.run(["ldd", str(rlk.LIB_PATH)], capture_output=True, text=True).stdout
    assert "oracle" not in deps


def desc(**kw):
    base = dict(num_tokens=4, real_vocab=1000, padded_vocab=1024, ld_logits=1024,
                num_vocab_tiles=64, num_virtual_shards=1, ignore_index=-100, validate=False)
    base.update(kw)
    return rlk.make_desc(**base)


def test_workspace_bytes():
    d = desc(num_tokens=32, num_vocab_tiles=64)
    part = (32 * 64 * 4 + 255) // 256 * 256
    assert rlk.rlk_logp_workspace_bytes(d) == 256 + 2 * part
    d = desc(num_tokens=3, num_vocab_tiles=5)
    assert rlk.rlk_logp_workspace_bytes(d) == 256 + 2 * 256
    assert rlk.rlk_logp_workspace_bytes(desc(num_tokens=0)) == 256
    assert rlk.rlk_logp_workspace_bytes(desc(num_vocab_tiles=0)) == 0


BAD_DESCS = [
    (dict(num_tokens=-1), rlk.RLK_ERR_BAD_SHAPE),
    (dict(num_tokens=2 ** 31), rlk.RLK_ERR_BAD_SHAPE),
    (dict(real_vocab=0), rlk.RLK_ERR_BAD_SHAPE),
    (dict(real_vocab=2000), rlk.RLK_ERR_BAD_SHAPE),  # > padded
    (dict(padded_vocab=2 ** 31, ld_logits=2 ** 31), rlk.RLK_ERR_BAD_SHAPE),
    (dict(ld_logits=1016), rlk.RLK_ERR_BAD_SHAPE),  # < padded
    (dict(ld_logits=1028), rlk.RLK_ERR_ALIGNMENT),
    (dict(num_vocab_tiles=0), rlk.RLK_ERR_BAD_TILING),
    (dict(num_vocab_tiles=1025), rlk.RLK_ERR_BAD_TILING),
    (dict(num_virtual_shards=0), rlk.RLK_ERR_BAD_TILING),
    (dict(num_virtual_shards=65), rlk.RLK_ERR_BAD_TILING),
]


@pytest.mark.parametrize("kw,code", BAD_DESCS)
def test_fwd_rejects_bad_descriptor_before_launch(kw, code):
    with pytest.raises(rlk.RlkError) as ei:
        rlk.rlk_logp_fwd(desc(**kw), None, None, None, None, None, None, stream=_NoStream())
    assert ei.value.status == code
    assert ei.value.detail


class _NoStream:
    """A stream stand-in: validation errors return before the stream is used."""
    cuda_stream = 0


class _FakeTensor:
    """A pointer stand-in (never dereferenced: every case fails validation first)."""

    def __init__(self, addr, nbytes=0):
        self.addr, self.nbytes = addr, nbytes

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1


def test_unknown_flags_and_null_desc():
    d = desc()
    d.flags = 0x80
    with pytest.raises(rlk.RlkError) as ei:
        rlk.rlk_logp_fwd(d, None, None, None, None, None, None, stream=_NoStream())
    assert ei.value.status == rlk.RLK_ERR_BAD_SHAPE
    lib = ctypes.CDLL(str(rlk.LIB_PATH))
    lib.rlk_logp_fwd.restype = ctypes.c_int
    assert lib.rlk_logp_fwd(None, None, None, None, None, None, None, ctypes.c_size_t(0),
                            None) == rlk.RLK_ERR_NULL_POINTER
    lib.rlk_logp_workspace_bytes.restype = ctypes.c_size_t
    assert lib.rlk_logp_workspace_bytes(None) == 0


def test_empty_batch_is_a_no_op():
    rlk.rlk_logp_fwd(desc(num_tokens=0), None, None, None, None, None, None, stream=_NoStream())
    rlk.rlk_logp_bwd(desc(num_tokens=0), None, None, None, None, None, None, 1024,
                     rlk.RLK_DTYPE_F32, None, stream=_NoStream())


def test_fwd_pointer_workspace_and_alignment_errors():
    d = desc()
    need = rlk.rlk_logp_workspace_bytes(d)
    a = _FakeTensor(0x10000000)
    ws = _FakeTensor(0x20000000, need)
    s = _NoStream()
    cases = [
        ((None, a, None, a, a, ws), rlk.RLK_ERR_NULL_POINTER),
        ((a, None, None, a, a, ws), rlk.RLK_ERR_NULL_POINTER),
        ((a, a, None, None, a, ws), rlk.RLK_ERR_NULL_POINTER),
        ((a, a, None, a, a, None), rlk.RLK_ERR_WORKSPACE),
        ((a, a, None, a, a, _FakeTensor(0x20000000, need - 1)), rlk.RLK_ERR_WORKSPACE),
        ((_FakeTensor(0x10000008), a, None, a, a, ws), rlk.RLK_ERR_ALIGNMENT),
        ((a, a, None, a, a, _FakeTensor(0x20000080, need)), rlk.RLK_ERR_ALIGNMENT),
        ((a, _FakeTensor(0x10000002), None, a, a, ws), rlk.RLK_ERR_ALIGNMENT),
    ]
    for args, code in cases:
        with pytest.raises(rlk.RlkError) as ei:
            rlk.rlk_logp_fwd(d, *args, stream=s)
        assert ei.value.status == code, (args, ei.value)


def test_bwd_argument_errors():
    d = desc()
    a = _FakeTensor(0x10000000)
    ws = _FakeTensor(0x20000000, 256)
    s = _NoStream()
    cases = [
        (dict(ld=1024, dt=7), rlk.RLK_ERR_DTYPE),
        (dict(ld=1016, dt=rlk.RLK_DTYPE_F32), rlk.RLK_ERR_BAD_SHAPE),
        (dict(ld=1028, dt=rlk.RLK_DTYPE_BF16), rlk.RLK_ERR_ALIGNMENT),
    ]
    for kw, code in cases:
        with pytest.raises(rlk.RlkError) as ei:
            rlk.rlk_logp_bwd(d, a, a, None, a, a, a, kw["ld"], kw["dt"], ws, stream=s)
        assert ei.value.status == code
    with pytest.raises(rlk.RlkError) as ei:
        rlk.rlk_logp_bwd(d, a, a, None, a, None, a, 1024, rlk.RLK_DTYPE_F32, ws, stream=s)
    assert ei.value.status == rlk.RLK_ERR_NULL_POINTER
    with pytest.raises(rlk.RlkError) as ei:
        rlk.rlk_logp_bwd(d, a, a, None, a, a, a, 1024, rlk.RLK_DTYPE_F32,
                         _FakeTensor(0x20000000, 255), stream=s)
    assert ei.value.status == rlk.RLK_ERR_WORKSPACE
    with pytest.raises(rlk.RlkError) as ei:
        rlk.rlk_logp_bwd(d, a, a, None, a, a, _FakeTensor(0x30000004), 1024, rlk.RLK_DTYPE_F32,
                         ws, stream=s)
    assert ei.value.status == rlk.RLK_ERR_ALIGNMENT


def test_status_strings():
    for code in range(10):
        assert rlk.rlk_status_string(code).startswith("RLK_")
    assert rlk.rlk_status_string(rlk.RLK_ERR_TARGET_RANGE) == "RLK_ERR_TARGET_RANGE"
    assert rlk.rlk_status_string(99) == "RLK_ERR_UNKNOWN"


@pytest.mark.parametrize("v_pad,t,s", [(151936, 64, 1), (152576, 64, 8), (10, 3, 2),
                                       (1000, 7, 3), (17, 17, 5), (5, 1, 1)])
def test_geometry_matches_oracle_and_pages(v_pad, t, s):
    bounds, first = rlk.rlk_logp_tile_geometry(v_pad, t, s)
    o = oracle.get()
    assert np.array_equal(np.array(bounds), o.tile_bounds(v_pad, t))
    assert np.array_equal(np.array(first), o.shard_tiles(t, s))
    if (v_pad, t) == (151936, 64):
        assert set(np.diff(bounds)) == {2374}
    if (v_pad, t) == (152576, 64):
        assert set(np.diff(bounds)) == {2384}


def test_geometry_errors():
    for args, code in (((0, 1, 1), rlk.RLK_ERR_BAD_SHAPE), ((10, 11, 1), rlk.RLK_ERR_BAD_TILING),
                       ((10, 4, 5), rlk.RLK_ERR_BAD_TILING)):
        with pytest.raises(rlk.RlkError) as ei:
            rlk.rlk_logp_tile_geometry(*args)
        assert ei.value.status == code


def test_fused_lmhead_host_validation():
    a = _FakeTensor(0x10000000)
    s = _NoStream()
    ok = desc(num_tokens=8, real_vocab=1000, padded_vocab=1024, num_vocab_tiles=4)
    need = rlk.rlk_logp_fused_lmhead_workspace_bytes(ok)
    n_vb = (1000 + 255) // 256
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert need == 256 + 2 * r(8 * 4 * 4) + r(8 * 4) + 2 * r(8 * 2 * n_vb * 4)
    ws = _FakeTensor(0x20000000, need)
    cases = [
        (desc(num_tokens=8, real_vocab=1000, padded_vocab=1024, num_vocab_tiles=5), 64,
         rlk.RLK_ERR_BAD_TILING),  # tiles narrower than 256 columns
        (desc(num_tokens=8, real_vocab=1000, padded_vocab=1024, num_vocab_tiles=4,
              num_virtual_shards=5), 64, rlk.RLK_ERR_BAD_TILING),  # more shards than tiles
        (desc(num_tokens=8, real_vocab=1000, padded_vocab=1024, num_vocab_tiles=4,
              num_virtual_shards=0), 64, rlk.RLK_ERR_BAD_TILING),
        (ok, 96, rlk.RLK_ERR_BAD_SHAPE),  # hidden_dim not a multiple of 64
        (ok, 0, rlk.RLK_ERR_BAD_SHAPE),
        (ok, (1 << 21) + 64, rlk.RLK_ERR_BAD_SHAPE),  # above 2^21
    ]
    for d, k, code in cases:
        with pytest.raises(rlk.RlkError) as ei:
            rlk.rlk_logp_fused_lmhead(d, a, a, k, a, None, a, a, ws, stream=s)
        assert ei.value.status == code, (k, ei.value)
    with pytest.raises(rlk.RlkError) as ei:
        rlk.rlk_logp_fused_lmhead(ok, a, a, 64, a, None, a, a, _FakeTensor(0x20000000, need - 1),
                                  stream=s)
    assert ei.value.status == rlk.RLK_ERR_WORKSPACE
    with pytest.raises(rlk.RlkError) as ei:
        rlk.rlk_logp_fused_lmhead(ok, _FakeTensor(0x10000004), a, 64, a, None, a, a, ws, stream=s)
    assert ei.value.status == rlk.RLK_ERR_ALIGNMENT
    with pytest.raises(rlk.RlkError) as ei:
        rlk.rlk_logp_fused_lmhead(ok, None, a, 64, a, None, a, a, ws, stream=s)
    assert ei.value.status == rlk.RLK_ERR_NULL_POINTER
    # an empty batch is a no-op
    rlk.rlk_logp_fused_lmhead(desc(num_tokens=0, real_vocab=1000, padded_vocab=1024,
                                   num_vocab_tiles=4), None, None, 64, None, None, None, None,
                              None, stream=s)


def test_fwd_bwd_host_validation():
    a = _FakeTensor(0x10000000)
    s = _NoStream()
    ok = desc(num_tokens=8, num_vocab_tiles=64)
    # the status words, plus one 64-bit partial slot per (row, tile) where the
    # unit schedule takes the geometry (T <= 64 tiles of 8 to about 2,500 columns)
    assert rlk.rlk_logp_fwd_bwd_workspace_bytes(ok) == 256 + 8 * 64 * 8
    assert rlk.rlk_logp_fwd_bwd_workspace_bytes(desc(num_vocab_tiles=1024)) == 256
    assert rlk.rlk_logp_fwd_bwd_workspace_bytes(desc(num_tokens=8, num_vocab_tiles=1)) == 256 + 64
    wide = desc(num_tokens=8, real_vocab=4000, padded_vocab=4096, ld_logits=4096,
                num_vocab_tiles=1)  # one 4096-column tile: 7 passes
    assert rlk.rlk_logp_fwd_bwd_workspace_bytes(wide) == 256
    # the row's partials live on chip: at most 1024 tiles
    big = desc(num_tokens=8, real_vocab=4000, padded_vocab=4096, ld_logits=4096,
               num_vocab_tiles=1025)
    assert rlk.rlk_logp_fwd_bwd_workspace_bytes(big) == 0
    ws = _FakeTensor(0x20000000, 256)
    f32 = rlk.RLK_DTYPE_F32

    def call(d=ok, logits=a, tgt=a, grad=a, logp=a, lse=a, dl=a, ld_d=1024, dt=f32, w=ws):
        with pytest.raises(rlk.RlkError) as ei:
            rlk.rlk_logp_fwd_bwd(d, logits, tgt, None, grad, logp, lse, dl, ld_d, dt, w, stream=s)
        return ei.value.status

    assert call(d=big) == rlk.RLK_ERR_BAD_TILING
    for kw, code in BAD_DESCS:
        assert call(d=desc(**kw)) == code, kw
    assert call(dt=7) == rlk.RLK_ERR_DTYPE
    assert call(ld_d=1016) == rlk.RLK_ERR_BAD_SHAPE
    assert call(ld_d=1028) == rlk.RLK_ERR_ALIGNMENT
    for name in ("logits", "tgt", "grad", "logp", "lse", "dl"):
        assert call(**{name: None}) == rlk.RLK_ERR_NULL_POINTER, name
    assert call(w=None) == rlk.RLK_ERR_WORKSPACE
    assert call(w=_FakeTensor(0x20000000, 255)) == rlk.RLK_ERR_WORKSPACE
    assert call(w=_FakeTensor(0x20000040, 256)) == rlk.RLK_ERR_ALIGNMENT
    assert call(logits=_FakeTensor(0x10000008)) == rlk.RLK_ERR_ALIGNMENT
    assert call(dl=_FakeTensor(0x30000004)) == rlk.RLK_ERR_ALIGNMENT
    assert call(grad=_FakeTensor(0x10000002)) == rlk.RLK_ERR_ALIGNMENT
    # an empty batch is a no-op
    rlk.rlk_logp_fwd_bwd(desc(num_tokens=0), None, None, None, None, None, None, None, 1024, f32,
                         None, stream=s)


def test_fwd_bwd_ex_host_validation():
    a = _FakeTensor(0x10000000)
    s = _NoStream()
    ok = desc(num_tokens=8, num_vocab_tiles=64)
    part = (8 * 64 * 4 + 255) // 256 * 256
    # the unit schedule's two slot arrays where the geometry fits, else the two
    # extended calls' workspace
    assert rlk.rlk_logp_fwd_bwd_ex_workspace_bytes(ok) == 256 + 2 * 8 * 64 * 8
    wide = desc(num_tokens=8, real_vocab=4000, padded_vocab=4096, ld_logits=4096,
                num_vocab_tiles=1)
    assert rlk.rlk_logp_fwd_bwd_ex_workspace_bytes(wide) == 256 + 3 * ((8 * 4 + 255) // 256 * 256)
    assert rlk.rlk_logp_fwd_bwd_ex_workspace_bytes(desc(num_vocab_tiles=1024)) == \
        rlk.rlk_logp_ex_workspace_bytes(desc(num_vocab_tiles=1024))
    assert rlk.rlk_logp_fwd_bwd_ex_workspace_bytes(desc(num_vocab_tiles=0)) == 0
    ws = _FakeTensor(0x20000000, 256 + 2 * 8 * 64 * 8)
    f32 = rlk.RLK_DTYPE_F32

    def call(d=ok, logits=a, tgt=a, g=a, gl=None, gh=None, logp=a, lse=a, ent=a, dl=a,
             ld_d=1024, dt=f32, w=ws):
        with pytest.raises(rlk.RlkError) as ei:
            rlk.rlk_logp_fwd_bwd_ex(d, logits, tgt, None, g, gl, gh, logp, lse, ent, dl, ld_d, dt,
                                    w, stream=s)
        return ei.value.status

    for kw, code in BAD_DESCS:
        assert call(d=desc(**kw)) == code, kw
    assert call(dt=7) == rlk.RLK_ERR_DTYPE
    assert call(ld_d=1016) == rlk.RLK_ERR_BAD_SHAPE
    assert call(ld_d=1028) == rlk.RLK_ERR_ALIGNMENT
    for name in ("logits", "tgt", "logp", "lse", "ent", "dl"):
        assert call(**{name: None}) == rlk.RLK_ERR_NULL_POINTER, name
    assert call(g=None) == rlk.RLK_ERR_NULL_POINTER  # no gradient at all
    assert call(w=None) == rlk.RLK_ERR_WORKSPACE
    # below the two calls' workspace (which is below the unit schedule's)
    assert call(w=_FakeTensor(0x20000000, 256 + 3 * part - 1)) == rlk.RLK_ERR_WORKSPACE
    assert call(w=_FakeTensor(0x20000040, 256 + 2 * 8 * 64 * 8)) == rlk.RLK_ERR_ALIGNMENT
    assert call(logits=_FakeTensor(0x10000008)) == rlk.RLK_ERR_ALIGNMENT
    assert call(gl=_FakeTensor(0x10000002)) == rlk.RLK_ERR_ALIGNMENT
    # an empty batch is a no-op
    rlk.rlk_logp_fwd_bwd_ex(desc(num_tokens=0), None, None, None, None, None, None, None, None,
                            None, None, 1024, f32, None, stream=s)


def test_extended_forward_and_backward_host_validation():
    a = _FakeTensor(0x10000000)
    s = _NoStream()
    d = desc(num_tokens=32, num_vocab_tiles=64)
    part = (32 * 64 * 4 + 255) // 256 * 256
    assert rlk.rlk_logp_ex_workspace_bytes(d) == 256 + 3 * part
    assert rlk.rlk_logp_ex_workspace_bytes(desc(num_vocab_tiles=0)) == 0
    need = 256 + 3 * part
    ws = _FakeTensor(0x20000000, need)

    def fwd(dd=d, ent=a, w=ws, logits=a):
        with pytest.raises(rlk.RlkError) as ei:
            rlk.rlk_logp_fwd_ex(dd, logits, a, None, a, a, ent, w, stream=s)
        return ei.value.status

    assert fwd(ent=None) == rlk.RLK_ERR_NULL_POINTER
    assert fwd(w=_FakeTensor(0x20000000, 256 + 2 * part)) == rlk.RLK_ERR_WORKSPACE
    assert fwd(logits=_FakeTensor(0x10000004)) == rlk.RLK_ERR_ALIGNMENT
    assert fwd(ent=_FakeTensor(0x10000002)) == rlk.RLK_ERR_ALIGNMENT
    for kw, code in BAD_DESCS:
        assert fwd(dd=desc(**kw)) == code, kw
    f32 = rlk.RLK_DTYPE_F32
    w256 = _FakeTensor(0x20000000, 256)

    def bwd(ent=a, g=a, gl=None, gh=None, dt=f32, ld_d=1024):
        with pytest.raises(rlk.RlkError) as ei:
            rlk.rlk_logp_bwd_ex(d, a, a, None, a, ent, g, gl, gh, a, ld_d, dt, w256, stream=s)
        return ei.value.status

    assert bwd(g=None) == rlk.RLK_ERR_NULL_POINTER  # no gradient at all
    assert bwd(ent=None, gh=a) == rlk.RLK_ERR_NULL_POINTER  # grad_ent needs entropy
    assert bwd(dt=3) == rlk.RLK_ERR_DTYPE
    assert bwd(ld_d=1020) == rlk.RLK_ERR_BAD_SHAPE
    assert bwd(gl=_FakeTensor(0x10000001)) == rlk.RLK_ERR_ALIGNMENT
    # empty batches are no-ops
    rlk.rlk_logp_fwd_ex(desc(num_tokens=0), None, None, None, None, None, None, None, stream=s)
    rlk.rlk_logp_bwd_ex(desc(num_tokens=0), None, None, None, None, None, None, None, None, None,
                        1024, f32, None, stream=s)


_LIMIT_PROBE = r"""
import ctypes, os, sys
lib = ctypes.CDLL(sys.argv[1])
fn = getattr(lib, "_ZN3rlk19launch_thread_limitEv")
fn.restype = ctypes.c_int64
first = fn()
os.environ["RLK_MAX_LAUNCH_THREADS"] = "2048"  # too late: read once per process
print(first, fn())
"""


def test_launch_thread_limit_reads_its_environment_variable_once():
    """The per-launch thread limit (a dispatch's grid size is 32 bits of threads): 2^31 by
    default, lowered by RLK_MAX_LAUNCH_THREADS (the hook the split-launch GPU test uses),
    never below 1024 threads, never above 2^31, a value that is not a number is ignored,
    and the variable is read once per process, at the first launch."""
    import os
    import subprocess
    import sys

    lib = ctypes.CDLL(str(rlk.LIB_PATH))
    if getattr(lib, "_ZN3rlk19launch_thread_limitEv", None) is None:
        pytest.skip("internal symbol not exported")
    for value, want in ((None, 1 << 31), ("5000", 5000), ("10", 1024), (str(1 << 40), 1 << 31),
                        ("abc", 1 << 31), ("", 1 << 31)):
        env = {k: v for k, v in os.environ.items() if k != "RLK_MAX_LAUNCH_THREADS"}
        if value is not None:
            env["RLK_MAX_LAUNCH_THREADS"] = value
        r = subprocess.run([sys.executable, "-c", _LIMIT_PROBE, str(rlk.LIB_PATH)], env=env,
                           capture_output=True, text=True, timeout=120, check=True)
        first, later = (int(x) for x in r.stdout.split())
        assert first == want and later == want, (value, r.stdout)


def test_conveniences_check_tensors_before_anything_runs():
    """The torch conveniences check each tensor's shape, dtype and device before calling the
    C entry points, which take bare pointers and cannot see dtypes (an int64 targets tensor
    would be read as pairs of int32 words)."""
    import torch

    n, v = 6, 40
    x = torch.zeros(n, v, dtype=torch.bfloat16)
    t32 = torch.zeros(n, dtype=torch.int32)
    g = torch.zeros(n)
    kw = dict(real_vocab=v, num_vocab_tiles=4)
    with pytest.raises(TypeError, match="int32"):
        rlk.forward(x, t32.long(), **kw)
    with pytest.raises(TypeError, match="bfloat16"):
        rlk.forward(x.float(), t32, **kw)
    with pytest.raises(ValueError, match="6 elements"):
        rlk.forward(x, t32[:5], **kw)
    with pytest.raises(ValueError, match="unit column stride"):
        rlk.forward(x.t(), t32, **kw)
    with pytest.raises(TypeError, match="active_mask"):
        rlk.forward(x, t32, torch.ones(n, dtype=torch.int32), **kw)
    with pytest.raises(TypeError, match="grad_logp"):
        rlk.backward(x, t32, None, g, g.double(), **kw)
    with pytest.raises(ValueError, match="contiguous"):
        rlk.backward(x, t32, None, torch.zeros(2 * n)[::2], g, **kw)
    with pytest.raises(TypeError, match="grad_logp"):
        rlk.forward_backward(x, t32, None, None, **kw)
    with pytest.raises(ValueError, match="GPU memory"):
        rlk.forward(x, t32, **kw)
    with pytest.raises(ValueError, match="columns"):
        rlk.fused_lmhead(torch.zeros(n, 64, dtype=torch.bfloat16),
                         torch.zeros(v, 128, dtype=torch.bfloat16), t32, real_vocab=v)
    with pytest.raises(ValueError, match="rows"):
        rlk.fused_lmhead(torch.zeros(n, 64, dtype=torch.bfloat16),
                         torch.zeros(v - 1, 64, dtype=torch.bfloat16), t32, real_vocab=v)
    with pytest.raises(TypeError, match="int32"):
        rlk.selected_token_logprob(x, t32.long(), real_vocab=v, num_vocab_tiles=4)
    # a view narrower than padded_vocab, or real_vocab beyond it, is refused before any
    # call: the kernels read columns [0, padded_vocab) of every row
    wide = torch.zeros(n, 2 * v, dtype=torch.bfloat16)
    narrow = wide[:, v // 2: v // 2 + v // 2]
    for call in (lambda **k: rlk.forward(narrow, t32, **k),
                 lambda **k: rlk.forward_ex(narrow, t32, **k),
                 lambda **k: rlk.backward(narrow, t32, None, g, g, **k),
                 lambda **k: rlk.backward_ex(narrow, t32, None, g, None, g, None, None, **k),
                 lambda **k: rlk.forward_backward(narrow, t32, None, g, **k),
                 lambda **k: rlk.selected_token_logprob(narrow, t32, **k)):
        with pytest.raises(ValueError, match="exceeds"):
            call(real_vocab=v // 2, padded_vocab=v, num_vocab_tiles=4)
        with pytest.raises(ValueError, match="exceeds"):
            call(real_vocab=v, num_vocab_tiles=4)  # real_vocab beyond the view's width
    with pytest.raises(ValueError, match="positive"):
        rlk.forward(x, t32, real_vocab=0, num_vocab_tiles=4)


def test_noalloc_forward_host_validation():
    """rlk_logp_fwd_noalloc: descriptor errors as rlk_logp_fwd; a problem whose
    workspace exceeds the fixed 32 MiB + 256 bytes scratch is refused with
    RLK_ERR_WORKSPACE before anything touches a device; an empty batch is a no-op."""
    import torch

    s = torch.cuda.current_stream() if torch.cuda.is_available() else None

    def call(d):
        return rlk._lib.rlk_logp_fwd_noalloc(ctypes.byref(d), None, None, None, None, None,
                                             None if s is None else s.cuda_stream)

    assert call(desc(num_vocab_tiles=0)) == rlk.RLK_ERR_BAD_TILING
    assert call(desc(num_tokens=-1)) == rlk.RLK_ERR_BAD_SHAPE
    assert call(desc(num_tokens=0)) == rlk.RLK_OK
    # 65,537 rows of 64 tiles need 256 + 2 * 16,777,472 bytes: one row too many
    big = desc(num_tokens=65537, real_vocab=151936, padded_vocab=152576, ld_logits=152576)
    assert rlk.rlk_logp_workspace_bytes(big) > (32 << 20) + 256
    assert call(big) == rlk.RLK_ERR_WORKSPACE
    assert "32" in rlk.rlk_last_error_detail() or "scratch" in rlk.rlk_last_error_detail()
    fits = desc(num_tokens=65536, real_vocab=151936, padded_vocab=152576, ld_logits=152576)
    assert rlk.rlk_logp_workspace_bytes(fits) == (32 << 20) + 256
    if not torch.cuda.is_available():  # no device to look the scratch up on
        assert call(fits) == rlk.RLK_ERR_HIP
