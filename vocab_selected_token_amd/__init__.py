"""Python binding of librlk_logp.so: deterministic selected-token logp on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/rlk_logp.h``; PyTorch supplies
device memory and the stream.  There is no fallback: if the library is not
built, importing this package raises.

Functions with the C names take caller-allocated tensors and mirror the C
signatures.  ``forward`` / ``backward`` are conveniences that allocate the
outputs and workspace with torch and call them.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "librlk_logp.so"

RLK_OK = 0
RLK_ERR_NULL_POINTER = 1
RLK_ERR_BAD_SHAPE = 2
RLK_ERR_BAD_TILING = 3
RLK_ERR_ALIGNMENT = 4
RLK_ERR_WORKSPACE = 5
RLK_ERR_DTYPE = 6
RLK_ERR_TARGET_RANGE = 7
RLK_ERR_NONFINITE_LSE = 8
RLK_ERR_HIP = 9

RLK_DTYPE_F32 = 0
RLK_DTYPE_BF16 = 1
RLK_FLAG_VALIDATE = 1

EXPORTED = ("rlk_logp_workspace_bytes", "rlk_logp_fwd", "rlk_logp_bwd",
            "rlk_logp_ex_workspace_bytes", "rlk_logp_fwd_ex", "rlk_logp_bwd_ex",
            "rlk_logp_fwd_bwd_workspace_bytes", "rlk_logp_fwd_bwd",
            "rlk_logp_fwd_bwd_ex_workspace_bytes", "rlk_logp_fwd_bwd_ex",
            "rlk_logp_fused_lmhead_workspace_bytes", "rlk_logp_fused_lmhead",
            "rlk_logp_tile_geometry", "rlk_status_string", "rlk_last_error_detail",
            "rlk_logp_fwd_noalloc")


class rlk_logp_desc(ctypes.Structure):  # noqa: N801 - mirrors the C struct name
    _fields_ = [("num_tokens", ctypes.c_int64), ("real_vocab", ctypes.c_int64),
                ("padded_vocab", ctypes.c_int64), ("ld_logits", ctypes.c_int64),
                ("num_vocab_tiles", ctypes.c_int32), ("num_virtual_shards", ctypes.c_int32),
                ("ignore_index", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class RlkError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{_lib.rlk_status_string(status).decode()}: {detail}")


def _load() -> ctypes.CDLL:
    if not LIB_PATH.exists():
        raise ImportError(f"{LIB_PATH} is not built; run vocab_selected_token_amd.build_lib "
                          "(there is no fallback path)")
    lib = ctypes.CDLL(str(LIB_PATH))
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    dp = ctypes.POINTER(rlk_logp_desc)
    lib.rlk_logp_workspace_bytes.argtypes = [dp]
    lib.rlk_logp_workspace_bytes.restype = sz
    lib.rlk_logp_fwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.rlk_logp_fwd.restype = ctypes.c_int
    lib.rlk_logp_fwd_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp]
    lib.rlk_logp_fwd_noalloc.restype = ctypes.c_int
    lib.rlk_logp_bwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, i64, ctypes.c_int, vp, sz, vp]
    lib.rlk_logp_bwd.restype = ctypes.c_int
    lib.rlk_logp_ex_workspace_bytes.argtypes = [dp]
    lib.rlk_logp_ex_workspace_bytes.restype = sz
    lib.rlk_logp_fwd_ex.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.rlk_logp_fwd_ex.restype = ctypes.c_int
    lib.rlk_logp_bwd_ex.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, ctypes.c_int, vp,
                                    sz, vp]
    lib.rlk_logp_bwd_ex.restype = ctypes.c_int
    lib.rlk_logp_fwd_bwd_workspace_bytes.argtypes = [dp]
    lib.rlk_logp_fwd_bwd_workspace_bytes.restype = sz
    lib.rlk_logp_fwd_bwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, i64, ctypes.c_int, vp, sz,
                                     vp]
    lib.rlk_logp_fwd_bwd.restype = ctypes.c_int
    lib.rlk_logp_fwd_bwd_ex_workspace_bytes.argtypes = [dp]
    lib.rlk_logp_fwd_bwd_ex_workspace_bytes.restype = sz
    lib.rlk_logp_fwd_bwd_ex.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64,
                                        ctypes.c_int, vp, sz, vp]
    lib.rlk_logp_fwd_bwd_ex.restype = ctypes.c_int
    lib.rlk_logp_fused_lmhead_workspace_bytes.argtypes = [dp]
    lib.rlk_logp_fused_lmhead_workspace_bytes.restype = sz
    lib.rlk_logp_fused_lmhead.argtypes = [dp, vp, vp, i64, vp, vp, vp, vp, vp, sz, vp]
    lib.rlk_logp_fused_lmhead.restype = ctypes.c_int
    lib.rlk_logp_tile_geometry.argtypes = [i64, i32, i32, vp, vp]
    lib.rlk_logp_tile_geometry.restype = ctypes.c_int
    lib.rlk_status_string.argtypes = [ctypes.c_int]
    lib.rlk_status_string.restype = ctypes.c_char_p
    lib.rlk_last_error_detail.argtypes = []
    lib.rlk_last_error_detail.restype = ctypes.c_char_p
    return lib


_lib = _load()


def _check(status: int) -> None:
    if status != RLK_OK:
        raise RlkError(status, _lib.rlk_last_error_detail().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_desc(num_tokens: int, real_vocab: int, padded_vocab: int, ld_logits: int,
              num_vocab_tiles: int = 64, num_virtual_shards: int = 1, ignore_index: int = -100,
              validate: bool = False) -> rlk_logp_desc:
    """The rlk_logp_desc of a call: ld_logits is the row stride of the logits in
    elements; validate sets RLK_FLAG_VALIDATE."""
    return rlk_logp_desc(num_tokens, real_vocab, padded_vocab, ld_logits, num_vocab_tiles,
                         num_virtual_shards, ignore_index,
                         RLK_FLAG_VALIDATE if validate else 0)


# -- the C entry points --------------------------------------------------------
# Each function below calls the C function of the same name (include/rlk_logp.h)
# with the same arguments in the same order: tensors go as their data pointers
# (None as NULL), a workspace tensor also gives its size in bytes, `stream`
# defaults to torch's current stream, and a status other than RLK_OK raises
# RlkError with the library's detail text.
def rlk_logp_workspace_bytes(desc: rlk_logp_desc) -> int:
    return int(_lib.rlk_logp_workspace_bytes(ctypes.byref(desc)))


def rlk_logp_fwd(desc, logits, targets, active_mask, logp, lse, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.rlk_logp_fwd(ctypes.byref(desc), _ptr(logits), _ptr(targets), _ptr(active_mask),
                             _ptr(logp), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def rlk_logp_fwd_noalloc(desc, logits, targets, active_mask, logp, lse, stream=None) -> None:
    _check(_lib.rlk_logp_fwd_noalloc(ctypes.byref(desc), _ptr(logits), _ptr(targets),
                                     _ptr(active_mask), _ptr(logp), _ptr(lse), _stream(stream)))


def rlk_logp_bwd(desc, logits, targets, active_mask, lse, grad_logp, dlogits, ld_dlogits: int,
                 dlogits_dtype: int, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.rlk_logp_bwd(ctypes.byref(desc), _ptr(logits), _ptr(targets), _ptr(active_mask),
                             _ptr(lse), _ptr(grad_logp), _ptr(dlogits), ld_dlogits,
                             dlogits_dtype, _ptr(workspace), ws_bytes, _stream(stream)))


def rlk_logp_ex_workspace_bytes(desc: rlk_logp_desc) -> int:
    return int(_lib.rlk_logp_ex_workspace_bytes(ctypes.byref(desc)))


def rlk_logp_fwd_ex(desc, logits, targets, active_mask, logp, lse, entropy, workspace,
                    stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.rlk_logp_fwd_ex(ctypes.byref(desc), _ptr(logits), _ptr(targets),
                                _ptr(active_mask), _ptr(logp), _ptr(lse), _ptr(entropy),
                                _ptr(workspace), ws_bytes, _stream(stream)))


def rlk_logp_bwd_ex(desc, logits, targets, active_mask, lse, entropy, grad_logp, grad_lse,
                    grad_ent, dlogits, ld_dlogits: int, dlogits_dtype: int, workspace,
                    stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.rlk_logp_bwd_ex(ctypes.byref(desc), _ptr(logits), _ptr(targets),
                                _ptr(active_mask), _ptr(lse), _ptr(entropy), _ptr(grad_logp),
                                _ptr(grad_lse), _ptr(grad_ent), _ptr(dlogits), ld_dlogits,
                                dlogits_dtype, _ptr(workspace), ws_bytes, _stream(stream)))


def rlk_logp_fwd_bwd_workspace_bytes(desc: rlk_logp_desc) -> int:
    return int(_lib.rlk_logp_fwd_bwd_workspace_bytes(ctypes.byref(desc)))


def rlk_logp_fwd_bwd(desc, logits, targets, active_mask, grad_logp, logp, lse, dlogits,
                     ld_dlogits: int, dlogits_dtype: int, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.rlk_logp_fwd_bwd(ctypes.byref(desc), _ptr(logits), _ptr(targets),
                                 _ptr(active_mask), _ptr(grad_logp), _ptr(logp), _ptr(lse),
                                 _ptr(dlogits), ld_dlogits, dlogits_dtype, _ptr(workspace),
                                 ws_bytes, _stream(stream)))


def rlk_logp_fwd_bwd_ex_workspace_bytes(desc: rlk_logp_desc) -> int:
    return int(_lib.rlk_logp_fwd_bwd_ex_workspace_bytes(ctypes.byref(desc)))


def rlk_logp_fwd_bwd_ex(desc, logits, targets, active_mask, grad_logp, grad_lse, grad_ent, logp,
                        lse, entropy, dlogits, ld_dlogits: int, dlogits_dtype: int, workspace,
                        stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.rlk_logp_fwd_bwd_ex(ctypes.byref(desc), _ptr(logits), _ptr(targets),
                                    _ptr(active_mask), _ptr(grad_logp), _ptr(grad_lse),
                                    _ptr(grad_ent), _ptr(logp), _ptr(lse), _ptr(entropy),
                                    _ptr(dlogits), ld_dlogits, dlogits_dtype, _ptr(workspace),
                                    ws_bytes, _stream(stream)))


def rlk_logp_fused_lmhead_workspace_bytes(desc: rlk_logp_desc) -> int:
    return int(_lib.rlk_logp_fused_lmhead_workspace_bytes(ctypes.byref(desc)))


def rlk_logp_fused_lmhead(desc, hidden, weight, hidden_dim: int, targets, active_mask, logp, lse,
                          workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.rlk_logp_fused_lmhead(ctypes.byref(desc), _ptr(hidden), _ptr(weight), hidden_dim,
                                      _ptr(targets), _ptr(active_mask), _ptr(logp), _ptr(lse),
                                      _ptr(workspace), ws_bytes, _stream(stream)))


def rlk_logp_tile_geometry(padded_vocab: int, num_vocab_tiles: int, num_virtual_shards: int = 1):
    """Host-only: (tile bounds [T+1] int64, shard first tiles [S+1] int32) as lists."""
    b = (ctypes.c_int64 * (num_vocab_tiles + 1))() if num_vocab_tiles >= 1 else None
    f = (ctypes.c_int32 * (num_virtual_shards + 1))() if num_virtual_shards >= 1 else None
    _check(_lib.rlk_logp_tile_geometry(padded_vocab, num_vocab_tiles, num_virtual_shards,
                                       ctypes.cast(b, ctypes.c_void_p) if b else None,
                                       ctypes.cast(f, ctypes.c_void_p) if f else None))
    return list(b), list(f)


def rlk_status_string(status: int) -> str:
    return _lib.rlk_status_string(status).decode()


def rlk_last_error_detail() -> str:
    return _lib.rlk_last_error_detail().decode()


# -- conveniences: allocate outputs with torch, then call the C entry points ----
# The C entry points take bare pointers and cannot see dtypes, so the conveniences
# check every tensor first (shape and dtype, then device) and raise before anything
# is enqueued.  Targets must already be int32: an int64 tensor would be read as
# pairs of int32 words, and narrowing it here could turn an out-of-range target
# into a valid column.
def _check_logits(logits, name="logits"):
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    if logits.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {logits.dtype}")
    if logits.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")


def _check_rows(name, t, n, dtypes):
    """A per-row vector: 1-D, n elements, contiguous, of one of `dtypes`."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        hint = " (convert with .to(torch.int32))" if name == "targets" else ""
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, "
                        f"got {t.dtype}{hint}")
    if t.dim() != 1 or t.numel() != n:
        raise ValueError(f"{name} must be 1-D with {n} elements, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_device(base, **tensors):
    if base.device.type != "cuda":
        raise ValueError(f"the inputs must be in GPU memory, got {base.device}")
    for name, t in tensors.items():
        if t is not None and t.device != base.device:
            raise ValueError(f"{name} is on {t.device}, the logits on {base.device}")


_F32 = (torch.float32,)
_I32 = (torch.int32,)
_MASK = (torch.uint8, torch.bool)


def _check_inputs(logits, targets, active_mask, **vectors):
    """logits bf16 [N, ld]; targets int32 [N]; mask uint8/bool [N] or None; every other
    keyword an fp32 [N] vector or None.  All on the logits' GPU."""
    _check_logits(logits)
    n = logits.shape[0]
    _check_rows("targets", targets, n, _I32)
    if targets is None:
        raise TypeError("targets must be a torch.Tensor")
    _check_rows("active_mask", active_mask, n, _MASK)
    for name, t in vectors.items():
        _check_rows(name, t, n, _F32)
    _check_device(logits, targets=targets, active_mask=active_mask, **vectors)


def _check_vocab(logits, real_vocab, padded_vocab):
    """The kernels read columns [0, V_pad) of every row (V_pad = padded_vocab, or the
    logits' width): a view narrower than that would let them read past it."""
    import operator
    _check_logits(logits)
    v_pad = operator.index(padded_vocab) if padded_vocab else logits.shape[1]
    if operator.index(real_vocab) < 1:
        raise ValueError(f"real_vocab must be positive, got {real_vocab!r}")
    if v_pad > logits.shape[1]:
        raise ValueError(f"padded_vocab={v_pad} exceeds the {logits.shape[1]} columns of the "
                         "logits")
    if real_vocab > v_pad:
        raise ValueError(f"real_vocab={real_vocab} exceeds padded_vocab={v_pad}")
    return v_pad


def _u8_mask(mask):
    if mask is None:
        return None
    return mask.view(torch.uint8) if mask.dtype == torch.bool else mask


def workspace_for(desc: rlk_logp_desc, device) -> torch.Tensor:
    """A fresh workspace of rlk_logp_workspace_bytes(desc) bytes for rlk_logp_fwd
    (its contents on entry do not matter)."""
    n = rlk_logp_workspace_bytes(desc)
    if n == 0:
        raise ValueError(f"invalid rlk_logp_desc: {rlk_last_error_detail()}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def forward(logits: torch.Tensor, targets: torch.Tensor, active_mask=None, *, real_vocab: int,
            padded_vocab: int | None = None, num_vocab_tiles: int = 64,
            num_virtual_shards: int = 1, ignore_index: int = -100, validate: bool = False,
            workspace: torch.Tensor | None = None, stream=None):
    """(logp, lse), fp32 [N] each.  logits: bf16 [N, ld] with unit column stride."""
    _check_vocab(logits, real_vocab, padded_vocab)
    _check_inputs(logits, targets, active_mask)
    n = logits.shape[0]
    desc = make_desc(n, real_vocab, padded_vocab or logits.shape[1], logits.stride(0),
                     num_vocab_tiles, num_virtual_shards, ignore_index, validate)
    logp = torch.empty(n, dtype=torch.float32, device=logits.device)
    lse = torch.empty(n, dtype=torch.float32, device=logits.device)
    if workspace is None:
        workspace = workspace_for(desc, logits.device)
    rlk_logp_fwd(desc, logits, targets, _u8_mask(active_mask), logp, lse, workspace, stream)
    return logp, lse


def backward(logits: torch.Tensor, targets: torch.Tensor, active_mask, lse: torch.Tensor,
             grad_logp: torch.Tensor, *, real_vocab: int, padded_vocab: int | None = None,
             out_dtype=torch.float32, ignore_index: int = -100, validate: bool = False,
             num_vocab_tiles: int | None = None, workspace: torch.Tensor | None = None,
             stream=None):
    """dlogits [N, V_pad] (fp32 or bf16)."""
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dlogits dtype must be torch.float32 or torch.bfloat16")
    _check_vocab(logits, real_vocab, padded_vocab)
    _check_inputs(logits, targets, active_mask, lse=lse, grad_logp=grad_logp)
    n = logits.shape[0]
    v_pad = padded_vocab or logits.shape[1]
    tiles = num_vocab_tiles if num_vocab_tiles is not None else min(64, v_pad)
    desc = make_desc(n, real_vocab, v_pad, logits.stride(0), tiles, 1, ignore_index, validate)
    ld_d = (v_pad + 7) // 8 * 8
    dl = torch.empty((n, ld_d), dtype=out_dtype, device=logits.device)
    if workspace is None:
        workspace = workspace_for(desc, logits.device)
    code = RLK_DTYPE_BF16 if out_dtype == torch.bfloat16 else RLK_DTYPE_F32
    rlk_logp_bwd(desc, logits, targets, _u8_mask(active_mask), lse, grad_logp, dl, ld_d, code,
                 workspace, stream)
    return dl[:, :v_pad]


def forward_ex(logits: torch.Tensor, targets: torch.Tensor, active_mask=None, *,
               real_vocab: int, padded_vocab: int | None = None, num_vocab_tiles: int = 64,
               num_virtual_shards: int = 1, ignore_index: int = -100, validate: bool = False,
               workspace: torch.Tensor | None = None, stream=None):
    """(logp, lse, entropy), fp32 [N] each."""
    _check_vocab(logits, real_vocab, padded_vocab)
    _check_inputs(logits, targets, active_mask)
    n = logits.shape[0]
    desc = make_desc(n, real_vocab, padded_vocab or logits.shape[1], logits.stride(0),
                     num_vocab_tiles, num_virtual_shards, ignore_index, validate)
    logp = torch.empty(n, dtype=torch.float32, device=logits.device)
    lse = torch.empty(n, dtype=torch.float32, device=logits.device)
    ent = torch.empty(n, dtype=torch.float32, device=logits.device)
    if workspace is None:
        nbytes = rlk_logp_ex_workspace_bytes(desc)
        if nbytes == 0:
            raise ValueError(f"invalid rlk_logp_desc: {rlk_last_error_detail()}")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=logits.device)
    rlk_logp_fwd_ex(desc, logits, targets, _u8_mask(active_mask), logp, lse, ent, workspace,
                    stream)
    return logp, lse, ent


def backward_ex(logits: torch.Tensor, targets: torch.Tensor, active_mask, lse: torch.Tensor,
                entropy=None, grad_logp=None, grad_lse=None, grad_ent=None, *, real_vocab: int,
                padded_vocab: int | None = None, out_dtype=torch.float32,
                ignore_index: int = -100, validate: bool = False,
                num_vocab_tiles: int | None = None, workspace: torch.Tensor | None = None,
                stream=None):
    """dlogits [N, V_pad] of a loss on (logp, lse, entropy); absent gradients are zero."""
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dlogits dtype must be torch.float32 or torch.bfloat16")
    _check_vocab(logits, real_vocab, padded_vocab)
    _check_inputs(logits, targets, active_mask, lse=lse, entropy=entropy, grad_logp=grad_logp,
                  grad_lse=grad_lse, grad_ent=grad_ent)
    n = logits.shape[0]
    v_pad = padded_vocab or logits.shape[1]
    tiles = num_vocab_tiles if num_vocab_tiles is not None else min(64, v_pad)
    desc = make_desc(n, real_vocab, v_pad, logits.stride(0), tiles, 1, ignore_index, validate)
    ld_d = (v_pad + 7) // 8 * 8
    dl = torch.empty((n, ld_d), dtype=out_dtype, device=logits.device)
    if workspace is None:
        workspace = workspace_for(desc, logits.device)
    code = RLK_DTYPE_BF16 if out_dtype == torch.bfloat16 else RLK_DTYPE_F32
    rlk_logp_bwd_ex(desc, logits, targets, _u8_mask(active_mask), lse, entropy, grad_logp,
                    grad_lse, grad_ent, dl, ld_d, code, workspace, stream)
    return dl[:, :v_pad]


class _SelectedTokenLogprob(torch.autograd.Function):
    """(logp, lse, entropy) of bf16 logits, differentiable in all three; the forward
    and the backward are rlk_logp_fwd_ex and rlk_logp_bwd_ex."""

    @staticmethod
    def forward(ctx, logits, targets, active_mask, real_vocab, padded_vocab, num_vocab_tiles,
                ignore_index):
        logp, lse, ent = forward_ex(logits, targets, active_mask, real_vocab=real_vocab,
                                    padded_vocab=padded_vocab, num_vocab_tiles=num_vocab_tiles,
                                    ignore_index=ignore_index)
        ctx.save_for_backward(logits, targets, lse, ent)
        ctx.active_mask = active_mask
        ctx.cfg = (real_vocab, padded_vocab, num_vocab_tiles, ignore_index)
        return logp, lse, ent

    @staticmethod
    def backward(ctx, g_logp, g_lse, g_ent):
        logits, targets, lse, ent = ctx.saved_tensors
        real_vocab, padded_vocab, num_vocab_tiles, ignore_index = ctx.cfg

        def vec(t):
            return None if t is None else t.contiguous().float()
        g_logp, g_lse, g_ent = vec(g_logp), vec(g_lse), vec(g_ent)
        if g_logp is None and g_lse is None and g_ent is None:
            return (None,) * 7
        v_pad = padded_vocab or logits.shape[1]
        d = backward_ex(logits, targets, ctx.active_mask, lse, ent, g_logp, g_lse, g_ent,
                        real_vocab=real_vocab, padded_vocab=v_pad, out_dtype=logits.dtype,
                        ignore_index=ignore_index, num_vocab_tiles=num_vocab_tiles)
        if d.shape == logits.shape and d.is_contiguous():
            grad = d
        else:
            grad = torch.zeros_like(logits)
            grad[:, :v_pad] = d
        return grad, None, None, None, None, None, None


def selected_token_logprob(logits: torch.Tensor, targets: torch.Tensor, active_mask=None, *,
                           real_vocab: int, padded_vocab: int | None = None,
                           num_vocab_tiles: int = 64, ignore_index: int = -100):
    """The op as a differentiable torch function: returns (logp, lse, entropy), fp32 [N].

    This is the interface a loss built on the selected-token log-probability
    consumes (a policy-gradient loss on logp, a penalty on LSE, an entropy bonus):
    autograd hands the three upstream gradients to rlk_logp_bwd_ex.  logits is
    bf16 [N, ld] with unit column stride; its gradient has its dtype.
    """
    _check_vocab(logits, real_vocab, padded_vocab)
    _check_inputs(logits, targets, active_mask)
    return _SelectedTokenLogprob.apply(logits, targets, active_mask, real_vocab, padded_vocab,
                                       num_vocab_tiles, ignore_index)


def forward_backward(logits: torch.Tensor, targets: torch.Tensor, active_mask,
                     grad_logp: torch.Tensor, *, real_vocab: int, padded_vocab: int | None = None,
                     num_vocab_tiles: int = 64, num_virtual_shards: int = 1,
                     out_dtype=torch.float32, ignore_index: int = -100, validate: bool = False,
                     workspace: torch.Tensor | None = None, stream=None):
    """(logp, lse, dlogits [N, V_pad]) in one launch, with g known up front.

    Bitwise the outputs of forward() then backward().  With the default workspace
    (rlk_logp_fwd_bwd_workspace_bytes) the unit schedule runs where the geometry
    takes it (T <= 64 tiles of 8 to about 2,500 columns): blocks of 8 tiles keep
    their logits on chip and exchange partials through the workspace; a
    256-byte workspace selects one block per row."""
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dlogits dtype must be torch.float32 or torch.bfloat16")
    if grad_logp is None:
        raise TypeError("grad_logp must be a torch.Tensor")
    _check_vocab(logits, real_vocab, padded_vocab)
    _check_inputs(logits, targets, active_mask, grad_logp=grad_logp)
    n = logits.shape[0]
    v_pad = padded_vocab or logits.shape[1]
    desc = make_desc(n, real_vocab, v_pad, logits.stride(0), num_vocab_tiles, num_virtual_shards,
                     ignore_index, validate)
    ld_d = (v_pad + 7) // 8 * 8
    logp = torch.empty(n, dtype=torch.float32, device=logits.device)
    lse = torch.empty(n, dtype=torch.float32, device=logits.device)
    dl = torch.empty((n, ld_d), dtype=out_dtype, device=logits.device)
    if workspace is None:
        nbytes = rlk_logp_fwd_bwd_workspace_bytes(desc)
        if nbytes == 0:
            raise ValueError(f"invalid rlk_logp_desc: {rlk_last_error_detail()}")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=logits.device)
    code = RLK_DTYPE_BF16 if out_dtype == torch.bfloat16 else RLK_DTYPE_F32
    rlk_logp_fwd_bwd(desc, logits, targets, _u8_mask(active_mask), grad_logp, logp, lse, dl, ld_d,
                     code, workspace, stream)
    return logp, lse, dl[:, :v_pad]


def forward_backward_ex(logits: torch.Tensor, targets: torch.Tensor, active_mask,
                        grad_logp=None, grad_lse=None, grad_ent=None, *, real_vocab: int,
                        padded_vocab: int | None = None, num_vocab_tiles: int = 64,
                        num_virtual_shards: int = 1, out_dtype=torch.float32,
                        ignore_index: int = -100, validate: bool = False,
                        workspace: torch.Tensor | None = None, stream=None):
    """(logp, lse, entropy, dlogits [N, V_pad]): forward_ex() then backward_ex() in one
    launch where the unit schedule takes the geometry (the same bits either way);
    absent gradients are zero, at least one must be given."""
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dlogits dtype must be torch.float32 or torch.bfloat16")
    _check_vocab(logits, real_vocab, padded_vocab)
    _check_inputs(logits, targets, active_mask, grad_logp=grad_logp, grad_lse=grad_lse,
                  grad_ent=grad_ent)
    n = logits.shape[0]
    v_pad = padded_vocab or logits.shape[1]
    desc = make_desc(n, real_vocab, v_pad, logits.stride(0), num_vocab_tiles, num_virtual_shards,
                     ignore_index, validate)
    ld_d = (v_pad + 7) // 8 * 8
    logp = torch.empty(n, dtype=torch.float32, device=logits.device)
    lse = torch.empty(n, dtype=torch.float32, device=logits.device)
    ent = torch.empty(n, dtype=torch.float32, device=logits.device)
    dl = torch.empty((n, ld_d), dtype=out_dtype, device=logits.device)
    if workspace is None:
        nbytes = rlk_logp_fwd_bwd_ex_workspace_bytes(desc)
        if nbytes == 0:
            raise ValueError(f"invalid rlk_logp_desc: {rlk_last_error_detail()}")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=logits.device)
    code = RLK_DTYPE_BF16 if out_dtype == torch.bfloat16 else RLK_DTYPE_F32
    rlk_logp_fwd_bwd_ex(desc, logits, targets, _u8_mask(active_mask), grad_logp, grad_lse,
                        grad_ent, logp, lse, ent, dl, ld_d, code, workspace, stream)
    return logp, lse, ent, dl[:, :v_pad]


def fused_lmhead(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                 active_mask=None, *, real_vocab: int, padded_vocab: int | None = None,
                 num_vocab_tiles: int = 64, num_virtual_shards: int = 1,
                 ignore_index: int = -100, validate: bool = False,
                 workspace: torch.Tensor | None = None, stream=None):
    """(logp, lse) of z = hidden . weight^T without materialising z.
    hidden: bf16 [N, K] contiguous; weight: bf16 [V_pad, K] contiguous."""
    for name, t in (("hidden", hidden), ("weight", weight)):
        _check_logits(t, name)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if weight.shape[1] != hidden.shape[1]:
        raise ValueError(f"weight has {weight.shape[1]} columns, hidden {hidden.shape[1]}")
    if weight.shape[0] < real_vocab:
        raise ValueError(f"weight has {weight.shape[0]} rows, fewer than real_vocab={real_vocab}")
    n = hidden.shape[0]
    _check_rows("targets", targets, n, _I32)
    if targets is None:
        raise TypeError("targets must be a torch.Tensor")
    _check_rows("active_mask", active_mask, n, _MASK)
    _check_device(hidden, weight=weight, targets=targets, active_mask=active_mask)
    n, k = hidden.shape
    v_pad = padded_vocab or weight.shape[0]
    desc = make_desc(n, real_vocab, v_pad, v_pad, num_vocab_tiles, num_virtual_shards,
                     ignore_index, validate)
    logp = torch.empty(n, dtype=torch.float32, device=hidden.device)
    lse = torch.empty(n, dtype=torch.float32, device=hidden.device)
    if workspace is None:
        nbytes = rlk_logp_fused_lmhead_workspace_bytes(desc)
        if nbytes == 0:
            raise ValueError(f"invalid rlk_logp_desc: {rlk_last_error_detail()}")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=hidden.device)
    rlk_logp_fused_lmhead(desc, hidden, weight, k, targets, _u8_mask(active_mask), logp, lse,
                          workspace, stream)
    return logp, lse
