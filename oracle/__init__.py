"""CPU oracle for selected-token log-probability (fp64, plain C).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg are the only callers.  The GPU library never imports, links or
executes anything here, and this package imports nothing from the library.

The arithmetic lives in ``rlk_oracle.c`` (see its header for the definitions
and the page passages each one follows).  This module only builds that file
with gcc, loads it with ctypes and marshals numpy arrays.

Parity pins: ``tests/test_oracle_pins.py`` checks every function here against
pure-Python brute force, closed forms, finite differences and float64 library
routines, and checks that deliberately broken builds of the C file fail them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SOURCE = HERE / "rlk_oracle.c"
LIB_PATH = HERE / "librlk_oracle.so"

ERR_ARG = 1
ERR_TARGET_RANGE = 2
ERR_NONFINITE_LSE = 3
ERR_NOMEM = 4

GCC_FLAGS = ["-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-Wextra"]


class OracleError(RuntimeError):
    def __init__(self, code: int, bad_row: int):
        self.code = code
        self.bad_row = bad_row
        name = {ERR_ARG: "bad argument", ERR_TARGET_RANGE: "active target out of range",
                ERR_NONFINITE_LSE: "non-finite LSE on an active row",
                ERR_NOMEM: "out of memory"}.get(code, f"code {code}")
        super().__init__(f"oracle: {name} (row {bad_row})")


def compile_oracle(src: Path, out: Path) -> Path:
    """Compile an oracle source with gcc (strict IEEE fp64: no fast-math, no contraction)."""
    tmp = out.with_name(f"{out.name}.tmp{os.getpid()}")  # parallel test workers may race
    subprocess.run(["gcc", *GCC_FLAGS, str(src), "-o", str(tmp), "-lpthread", "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> Path:
    if force or not LIB_PATH.exists():
        compile_oracle(SOURCE, LIB_PATH)
    return LIB_PATH


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logits(x):
    """Return (array, is_bf16): bf16 logits travel as their uint16 bit patterns."""
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("oracle logits must be 2-D [rows, ld]")
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), True
    if x.dtype == np.float64:
        return np.ascontiguousarray(x), False
    raise TypeError("oracle logits must be float64 or bf16 bit patterns (uint16)")


def _prep_rows(tgt, mask, n):
    tgt = np.ascontiguousarray(np.asarray(tgt, dtype=np.int32).reshape(-1))
    if tgt.shape[0] != n:
        raise ValueError("targets must have one entry per row")
    if mask is not None:
        mask = np.ascontiguousarray((np.asarray(mask).reshape(-1) != 0).astype(np.uint8))
        if mask.shape[0] != n:
            raise ValueError("mask must have one entry per row")
    return tgt, mask


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, lib_path: Path):
        lib = ctypes.CDLL(str(lib_path))
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        lib.rlk_oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.rlk_oracle_bf16_to_f64.restype = ctypes.c_double
        lib.rlk_oracle_tile_bounds.argtypes = [i64, i32, vp]
        lib.rlk_oracle_shard_tiles.argtypes = [i32, i32, vp]
        fwd_args = [vp, i64, i64, i64, vp, vp, i32, vp, vp, vp, ctypes.c_int]
        lib.rlk_oracle_fwd_f64.argtypes = fwd_args
        lib.rlk_oracle_fwd_bf16.argtypes = fwd_args
        bwd_args = [vp, i64, i64, i64, i64, vp, vp, i32, vp, vp, vp, i64, vp, ctypes.c_int]
        lib.rlk_oracle_bwd_f64.argtypes = bwd_args
        lib.rlk_oracle_bwd_bf16.argtypes = bwd_args
        part_args = [vp, i64, i64, i64, i64, i32, vp, vp, vp, ctypes.c_int]
        lib.rlk_oracle_tile_partials_f64.argtypes = part_args
        lib.rlk_oracle_tile_partials_bf16.argtypes = part_args
        ent_args = [vp, i64, i64, i64, vp, ctypes.c_int]
        lib.rlk_oracle_entropy_f64.argtypes = ent_args
        lib.rlk_oracle_entropy_bf16.argtypes = ent_args
        bwd_ex_args = [vp, i64, i64, i64, i64, vp, vp, i32, vp, vp, vp, vp, vp, vp, i64, vp,
                       ctypes.c_int]
        lib.rlk_oracle_bwd_ex_f64.argtypes = bwd_ex_args
        lib.rlk_oracle_bwd_ex_bf16.argtypes = bwd_ex_args
        lib.rlk_oracle_lmhead_logits.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp, ctypes.c_int]
        lib.rlk_oracle_lmhead_logits.restype = ctypes.c_int
        for name in ("rlk_oracle_tile_bounds", "rlk_oracle_shard_tiles", "rlk_oracle_fwd_f64",
                     "rlk_oracle_fwd_bf16", "rlk_oracle_bwd_f64", "rlk_oracle_bwd_bf16",
                     "rlk_oracle_tile_partials_f64", "rlk_oracle_tile_partials_bf16",
                     "rlk_oracle_entropy_f64", "rlk_oracle_entropy_bf16", "rlk_oracle_bwd_ex_f64",
                     "rlk_oracle_bwd_ex_bf16"):
            getattr(lib, name).restype = ctypes.c_int
        self._lib = lib
        self.path = Path(lib_path)

    # -- decoding and geometry ------------------------------------------------
    def bf16_to_f64(self, bits: int) -> float:
        return self._lib.rlk_oracle_bf16_to_f64(int(bits) & 0xFFFF)

    def tile_bounds(self, padded_vocab: int, num_tiles: int) -> np.ndarray:
        out = np.zeros(num_tiles + 1, dtype=np.int64)
        rc = self._lib.rlk_oracle_tile_bounds(padded_vocab, num_tiles, _ptr(out))
        if rc:
            raise OracleError(rc, -1)
        return out

    def shard_tiles(self, num_tiles: int, num_shards: int) -> np.ndarray:
        out = np.zeros(num_shards + 1, dtype=np.int32)
        rc = self._lib.rlk_oracle_shard_tiles(num_tiles, num_shards, _ptr(out))
        if rc:
            raise OracleError(rc, -1)
        return out

    # -- forward / backward ---------------------------------------------------
    def fwd(self, x, tgt, mask=None, *, real_vocab: int, ignore_index: int = -100,
            nthreads: int = 0, raise_on_error: bool = True):
        """Selected-token logp and LSE in fp64.  x: [N, ld] float64 or uint16 (bf16 bits).

        Returns (logp, lse, status, bad_row).  With raise_on_error a nonzero status raises.
        """
        x, is_bf16 = _logits(x)
        n, ld = x.shape
        tgt, mask = _prep_rows(tgt, mask, n)
        logp = np.empty(n, dtype=np.float64)
        lse = np.empty(n, dtype=np.float64)
        bad = ctypes.c_int64(-1)
        fn = self._lib.rlk_oracle_fwd_bf16 if is_bf16 else self._lib.rlk_oracle_fwd_f64
        rc = fn(_ptr(x), n, real_vocab, ld, _ptr(tgt), _ptr(mask), ignore_index,
                _ptr(logp), _ptr(lse), ctypes.byref(bad), nthreads)
        if rc == ERR_ARG or (rc and raise_on_error):
            raise OracleError(rc, bad.value)
        return logp, lse, rc, bad.value

    def bwd(self, x, tgt, mask, lse, g, *, real_vocab: int, padded_vocab: int,
            ignore_index: int = -100, nthreads: int = 0, raise_on_error: bool = True):
        """dlogits = g * (onehot - softmax) on effective-active rows, fp64 [N, padded_vocab]."""
        x, is_bf16 = _logits(x)
        n, ld = x.shape
        tgt, mask = _prep_rows(tgt, mask, n)
        lse = np.ascontiguousarray(np.asarray(lse, dtype=np.float64).reshape(-1))
        g = np.ascontiguousarray(np.asarray(g, dtype=np.float64).reshape(-1))
        d = np.empty((n, padded_vocab), dtype=np.float64)
        bad = ctypes.c_int64(-1)
        fn = self._lib.rlk_oracle_bwd_bf16 if is_bf16 else self._lib.rlk_oracle_bwd_f64
        rc = fn(_ptr(x), n, real_vocab, padded_vocab, ld, _ptr(tgt), _ptr(mask), ignore_index,
                _ptr(lse), _ptr(g), _ptr(d), padded_vocab, ctypes.byref(bad), nthreads)
        if rc == ERR_ARG or (rc and raise_on_error):
            raise OracleError(rc, bad.value)
        return d

    def entropy(self, x, *, real_vocab: int, nthreads: int = 0) -> np.ndarray:
        """H_r = -sum p log p over the real columns (fp64); NaN where LSE is not finite."""
        x, is_bf16 = _logits(x)
        n, ld = x.shape
        ent = np.empty(n, dtype=np.float64)
        fn = self._lib.rlk_oracle_entropy_bf16 if is_bf16 else self._lib.rlk_oracle_entropy_f64
        rc = fn(_ptr(x), n, real_vocab, ld, _ptr(ent), nthreads)
        if rc:
            raise OracleError(rc, -1)
        return ent

    def bwd_ex(self, x, tgt, mask, lse, *, real_vocab: int, padded_vocab: int, ent=None, g=None,
               g_lse=None, g_ent=None, ignore_index: int = -100, nthreads: int = 0,
               raise_on_error: bool = True):
        """d = a g (onehot - p) + g_lse p - g_ent p (log p + H), fp64 [N, padded_vocab].
        g, g_lse, g_ent may be None (zero); ent is needed when g_ent is given."""
        x, is_bf16 = _logits(x)
        n, ld = x.shape
        tgt, mask = _prep_rows(tgt, mask, n)

        def vec(v):
            return None if v is None else np.ascontiguousarray(
                np.asarray(v, dtype=np.float64).reshape(-1))
        lse, ent, g, g_lse, g_ent = vec(lse), vec(ent), vec(g), vec(g_lse), vec(g_ent)
        d = np.empty((n, padded_vocab), dtype=np.float64)
        bad = ctypes.c_int64(-1)
        fn = self._lib.rlk_oracle_bwd_ex_bf16 if is_bf16 else self._lib.rlk_oracle_bwd_ex_f64
        rc = fn(_ptr(x), n, real_vocab, padded_vocab, ld, _ptr(tgt), _ptr(mask), ignore_index,
                _ptr(lse), _ptr(ent), _ptr(g), _ptr(g_lse), _ptr(g_ent), _ptr(d), padded_vocab,
                ctypes.byref(bad), nthreads)
        if rc == ERR_ARG or (rc and raise_on_error):
            raise OracleError(rc, bad.value)
        return d

    def lmhead_logits(self, h, w, *, real_vocab: int, nthreads: int = 0) -> np.ndarray:
        """z = h . W^T in fp64 over W's first real_vocab rows.  h: [N, K], W: [V, K],
        both bf16 bit patterns (uint16).  Returns [N, real_vocab] float64."""
        h = np.ascontiguousarray(np.asarray(h))
        w = np.ascontiguousarray(np.asarray(w))
        if h.dtype != np.uint16 or w.dtype != np.uint16 or h.ndim != 2 or w.ndim != 2:
            raise TypeError("h and W must be 2-D bf16 bit patterns (uint16)")
        if h.shape[1] != w.shape[1] or w.shape[0] < real_vocab:
            raise ValueError("h [N, K] and W [>= real_vocab, K] must share K")
        n, k = h.shape
        z = np.empty((n, real_vocab), dtype=np.float64)
        rc = self._lib.rlk_oracle_lmhead_logits(_ptr(h), _ptr(w), n, k, real_vocab, k, k,
                                                _ptr(z), nthreads)
        if rc:
            raise OracleError(rc, -1)
        return z

    def lmhead_logits_blas(self, h, w, *, real_vocab: int) -> np.ndarray:
        """z = h . W^T over W's first real_vocab rows, as lmhead_logits computes it, with
        numpy's float64 matrix product as the one step (fast enough for the 4096-token
        workload in full; the plain-loop form pins it).  Decoding a bf16 pattern is exact:
        its 16 bits are the top half of an IEEE binary32."""
        h = np.ascontiguousarray(np.asarray(h))
        w = np.ascontiguousarray(np.asarray(w))
        if h.dtype != np.uint16 or w.dtype != np.uint16 or h.ndim != 2 or w.ndim != 2:
            raise TypeError("h and W must be 2-D bf16 bit patterns (uint16)")
        if h.shape[1] != w.shape[1] or w.shape[0] < real_vocab:
            raise ValueError("h [N, K] and W [>= real_vocab, K] must share K")
        hd = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        wd = (w[:real_vocab].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return hd @ wd.T

    def lmhead_fwd(self, h, w, tgt, mask=None, *, real_vocab: int, ignore_index: int = -100,
                   nthreads: int = 0, raise_on_error: bool = True):
        """Selected-token logp and LSE of z = h . W^T (fp64): (logp, lse, status, bad_row)."""
        z = self.lmhead_logits(h, w, real_vocab=real_vocab, nthreads=nthreads)
        return self.fwd(z, tgt, mask, real_vocab=real_vocab, ignore_index=ignore_index,
                        nthreads=nthreads, raise_on_error=raise_on_error)

    def tile_partials(self, x, *, real_vocab: int, padded_vocab: int, num_tiles: int,
                      nthreads: int = 0, with_entropy: bool = False):
        """Per-tile (max, sumexp) over each tile's real columns, fp64, each [N, T]; with
        with_entropy also the per-tile sum of exp(x - m) (x - m)."""
        x, is_bf16 = _logits(x)
        n, ld = x.shape
        pmax = np.empty((n, num_tiles), dtype=np.float64)
        psum = np.empty((n, num_tiles), dtype=np.float64)
        pent = np.empty((n, num_tiles), dtype=np.float64) if with_entropy else None
        fn = (self._lib.rlk_oracle_tile_partials_bf16 if is_bf16
              else self._lib.rlk_oracle_tile_partials_f64)
        rc = fn(_ptr(x), n, real_vocab, padded_vocab, ld, num_tiles, _ptr(pmax), _ptr(psum),
                _ptr(pent), nthreads)
        if rc:
            raise OracleError(rc, -1)
        return (pmax, psum, pent) if with_entropy else (pmax, psum)


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from rlk_oracle.c (rebuilt when the source is newer)."""
    global _default
    if _default is None:
        if not LIB_PATH.exists() or LIB_PATH.stat().st_mtime < SOURCE.stat().st_mtime:
            build(force=True)
        _default = Oracle(LIB_PATH)
    return _default
