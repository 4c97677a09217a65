"""Thin ctypes binding of libloglin.so (C ABI in include/loglin.h).

The functions carry the names of the C entry points and only marshal
arguments: they check that tensors are contiguous CUDA (HIP) tensors of the
right dtype and shape, allocate outputs and workspace with torch when the
caller passes none, and pass raw pointers plus torch's current stream.  All
arithmetic runs in the library's HIP kernels.  If the library is missing the
first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libloglin.so")

LOGLIN_OK, LOGLIN_EINVAL, LOGLIN_EUNSUPPORTED, LOGLIN_ENOMEM, LOGLIN_ECAPACITY, LOGLIN_EHIP = range(6)
LOGLIN_F32, LOGLIN_BF16 = 0, 1

_DTYPES = {torch.float32: LOGLIN_F32, torch.bfloat16: LOGLIN_BF16}


class LoglinError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class FwdPlan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("tile", ctypes.c_int), ("seg_tiles", ctypes.c_int),
                ("nseg", ctypes.c_int), ("col_block", ctypes.c_int),
                ("coarse_levels", ctypes.c_int), ("state_split", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t)]

    def as_dict(self) -> dict:
        d = {n: getattr(self, n) for n, _ in self._fields_}
        d["path"] = {0: "chunked", 1: "fused"}.get(self.path, str(self.path))
        return d


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -m log_linear_token_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.loglin_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.loglin_fwd_workspace_bytes.restype = sz
    lib.loglin_fwd_chunked.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.loglin_fwd_chunked.restype = i
    lib.loglin_fwd_chunked_stages.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp,
                                              sz, ctypes.c_uint, vp]
    lib.loglin_fwd_chunked_stages.restype = i
    lib.loglin_fwd_chunked_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp]
    lib.loglin_fwd_chunked_noalloc.restype = i
    lib.loglin_gdn_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.loglin_gdn_fwd_workspace_bytes.restype = sz
    lib.loglin_gdn_fwd_chunked_stages.argtypes = [vp] * 7 + [i] * 8 + [vp, sz, ctypes.c_uint, vp]
    lib.loglin_gdn_fwd_chunked_stages.restype = i
    lib.loglin_gdn_decode_step.argtypes = [vp] * 8 + [i, vp]
    lib.loglin_gdn_decode_step.restype = i
    lib.loglin_fwd_plan.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(FwdPlan)]
    lib.loglin_fwd_plan.restype = i
    lib.loglin_state_init.argtypes = [ctypes.POINTER(vp), i, i, i, i, i, vp]
    lib.loglin_state_init.restype = i
    lib.loglin_state_free.argtypes = [vp]
    lib.loglin_state_free.restype = i
    lib.loglin_state_load.argtypes = [vp, vp, vp, vp]
    lib.loglin_state_load.restype = i
    lib.loglin_state_export.argtypes = [vp, vp, vp, vp]
    lib.loglin_state_export.restype = i
    lib.loglin_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, vp]
    lib.loglin_decode_step.restype = i
    lib.loglin_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.loglin_bwd_workspace_bytes.restype = sz
    lib.loglin_bwd_chunked.argtypes = [vp] * 11 + [i] * 8 + [vp, sz, vp]
    lib.loglin_bwd_chunked.restype = i
    lib.loglin_prefill_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.loglin_prefill_workspace_bytes.restype = sz
    lib.loglin_prefill_states.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp, sz, vp]
    lib.loglin_prefill_states.restype = i
    lib.loglin_debug_level_map.argtypes = [i, vp, vp]
    lib.loglin_debug_level_map.restype = i
    lib.loglin_last_error.argtypes = []
    lib.loglin_last_error.restype = ctypes.c_char_p
    lib.loglin_status_string.argtypes = [i]
    lib.loglin_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _status_name(s: int) -> str:
    try:
        return _load().loglin_status_string(s).decode()
    except Exception:  # library not loadable: still produce a message
        return f"status {s}"


def loglin_last_error() -> str:
    return _load().loglin_last_error().decode()


def _check(rc: int) -> None:
    if rc != LOGLIN_OK:
        raise LoglinError(rc, loglin_last_error())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t.data_ptr()


# ---------------------------------------------------------------- forward

def _dt_code(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be torch.float32 or torch.bfloat16 (got {dtype})")
    return _DTYPES[dtype]


def loglin_fwd_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, C: int,
                               dtype=torch.bfloat16) -> int:
    n = _load().loglin_fwd_workspace_bytes(B, H, T, dk, dv, C, _dt_code(dtype))
    if n == ctypes.c_size_t(-1).value:
        raise LoglinError(LOGLIN_EINVAL, loglin_last_error())
    return n


def loglin_fwd_plan(B: int, H: int, T: int, dk: int, dv: int, C: int, dtype=torch.bfloat16) -> dict:
    pl = FwdPlan()
    _check(_load().loglin_fwd_plan(B, H, T, dk, dv, C, _dt_code(dtype), ctypes.byref(pl)))
    return pl.as_dict()


STAGE_CHUNK_STATE, STAGE_SCAN, STAGE_OUTPUT, STAGE_ALL = 1, 2, 4, 7


def loglin_fwd_chunked(q, k, v, log_decay, lam, C: int, out=None, workspace=None):
    """O = (Q K^T (.) M) V for the log-linear mask, chunked on the GPU.

    q, k [B,H,T,dk] and v [B,H,T,dv] (float32 or bfloat16, same dtype);
    log_decay [B,H,T] float32; lam [B,H,T,L] float32.  Returns out
    [B,H,T,dv] float32.
    """
    return loglin_fwd_chunked_stages(q, k, v, log_decay, lam, C, STAGE_ALL, out, workspace)


def loglin_fwd_chunked_stages(q, k, v, log_decay, lam, C: int, stage_mask: int, out=None,
                              workspace=None):
    """Profiling variant: enqueue only the kernels selected by stage_mask."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be float32 or bfloat16 (got {q.dtype})")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    pq = _dev(q, "q", q.dtype)
    pk = _dev(k, "k", q.dtype, (B, H, T, dk))
    pv = _dev(v, "v", q.dtype, (B, H, T, dv))
    pa = _dev(log_decay, "log_decay", torch.float32, (B, H, T))
    pl = _dev(lam, "lam", torch.float32, (B, H, T, L))
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=torch.float32, device=q.device)
    po = _dev(out, "out", torch.float32, (B, H, T, dv))
    need = loglin_fwd_workspace_bytes(B, H, T, dk, dv, C, q.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    pw = _dev(workspace, "workspace") if workspace is not None else None
    nws = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_load().loglin_fwd_chunked_stages(pq, pk, pv, pa, pl, po, B, H, T, dk, dv, L, C,
                                             _DTYPES[q.dtype], pw, nws, stage_mask, _stream(q)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # LOGLIN_NOALLOC_SCRATCH_BYTES


def loglin_fwd_chunked_noalloc(q, k, v, log_decay, lam, C: int, out=None):
    """loglin_fwd_chunked without a workspace argument: the library takes it
    from its own static device array (no device allocation in the call).
    `out` must be passed by callers that cannot allocate; when it is None it
    is allocated here, outside the library call."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be float32 or bfloat16 (got {q.dtype})")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    pq = _dev(q, "q", q.dtype)
    pk = _dev(k, "k", q.dtype, (B, H, T, dk))
    pv = _dev(v, "v", q.dtype, (B, H, T, dv))
    pa = _dev(log_decay, "log_decay", torch.float32, (B, H, T))
    pl = _dev(lam, "lam", torch.float32, (B, H, T, L))
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=torch.float32, device=q.device)
    po = _dev(out, "out", torch.float32, (B, H, T, dv))
    _check(_load().loglin_fwd_chunked_noalloc(pq, pk, pv, pa, pl, po, B, H, T, dk, dv, L, C,
                                              _DTYPES[q.dtype], _stream(q)))
    return out


# ---------------------------------------------------------------- Gated DeltaNet

def loglin_gdn_fwd_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, C: int,
                                   dtype=torch.bfloat16) -> int:
    n = _load().loglin_gdn_fwd_workspace_bytes(B, H, T, dk, dv, C, _dt_code(dtype))
    if n == ctypes.c_size_t(-1).value:
        raise LoglinError(LOGLIN_EUNSUPPORTED, loglin_last_error())
    return n


GDN_STAGE_CHUNK, GDN_STAGE_LEVELS, GDN_STAGE_ALL = 1, 2, 3


def loglin_gdn_fwd_chunked(q, k, v, log_decay, beta, lam, C: int, out=None, workspace=None,
                           stage_mask: int = GDN_STAGE_ALL):
    """Log-linear Gated DeltaNet forward: q, k [B,H,T,dk], v [B,H,T,dv] (float32
    or bfloat16), log_decay and beta [B,H,T] float32, lam [B,H,T,L] float32.
    Returns out [B,H,T,dv] float32."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be float32 or bfloat16 (got {q.dtype})")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    pq = _dev(q, "q", q.dtype)
    pk = _dev(k, "k", q.dtype, (B, H, T, dk))
    pv = _dev(v, "v", q.dtype, (B, H, T, dv))
    pa = _dev(log_decay, "log_decay", torch.float32, (B, H, T))
    pb = _dev(beta, "beta", torch.float32, (B, H, T))
    pl = _dev(lam, "lam", torch.float32, (B, H, T, L))
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=torch.float32, device=q.device)
    po = _dev(out, "out", torch.float32, (B, H, T, dv))
    need = loglin_gdn_fwd_workspace_bytes(B, H, T, dk, dv, C, q.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    pw = _dev(workspace, "workspace") if workspace is not None else None
    nws = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_load().loglin_gdn_fwd_chunked_stages(pq, pk, pv, pa, pb, pl, po, B, H, T, dk, dv, L, C,
                                                 _DTYPES[q.dtype], pw, nws, stage_mask, _stream(q)))
    return out


# ---------------------------------------------------------------- backward

def loglin_bwd_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, C: int,
                               dtype=torch.bfloat16) -> int:
    n = _load().loglin_bwd_workspace_bytes(B, H, T, dk, dv, C, _dt_code(dtype))
    if n == ctypes.c_size_t(-1).value:
        raise LoglinError(LOGLIN_EINVAL, loglin_last_error())
    return n


def loglin_bwd_chunked(q, k, v, log_decay, lam, dout, C: int, grads=None, workspace=None):
    """Gradients of sum(O * dout) for O = loglin_fwd_chunked(q, k, v, log_decay, lam, C).

    dout [B,H,T,dv] in the dtype of q.  Returns (dq, dk, dv, dlog_decay,
    dlam), all float32, shaped like q, k, v, log_decay and lam; `grads`
    may pass those five tensors in to be written.
    """
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be float32 or bfloat16 (got {q.dtype})")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    ptrs = [_dev(q, "q", q.dtype), _dev(k, "k", q.dtype, (B, H, T, dk)),
            _dev(v, "v", q.dtype, (B, H, T, dv)),
            _dev(log_decay, "log_decay", torch.float32, (B, H, T)),
            _dev(lam, "lam", torch.float32, (B, H, T, L)),
            _dev(dout, "dout", q.dtype, (B, H, T, dv))]
    shapes = [(B, H, T, dk), (B, H, T, dk), (B, H, T, dv), (B, H, T), (B, H, T, L)]
    names = ["dq", "dk", "dv", "dlog_decay", "dlam"]
    if grads is None:
        grads = tuple(torch.empty(sh, dtype=torch.float32, device=q.device) for sh in shapes)
    ptrs += [_dev(g, n, torch.float32, sh) for g, n, sh in zip(grads, names, shapes)]
    need = loglin_bwd_workspace_bytes(B, H, T, dk, dv, C, q.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    pw = _dev(workspace, "workspace") if workspace is not None else None
    nws = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_load().loglin_bwd_chunked(*ptrs, B, H, T, dk, dv, L, C, _DTYPES[q.dtype], pw, nws,
                                      _stream(q)))
    return tuple(grads)


# ---------------------------------------------------------------- prefill -> decode

def loglin_prefill_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, Lmax: int) -> int:
    n = _load().loglin_prefill_workspace_bytes(B, H, T, dk, dv, Lmax)
    if n == ctypes.c_size_t(-1).value:
        raise LoglinError(LOGLIN_EINVAL, loglin_last_error())
    return n


def loglin_prefill_states(k, v, log_decay, Lmax: int, out=None, workspace=None):
    """Fenwick level states after the T tokens of each sequence, in the layout
    loglin_state_load takes: k [B,H,T,dk], v [B,H,T,dv] (float32 or
    bfloat16), log_decay [B,H,T] float32.  Returns [B,H,Lmax,dk,dv] float32."""
    if k.dtype not in _DTYPES:
        raise ValueError(f"k must be float32 or bfloat16 (got {k.dtype})")
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    pk = _dev(k, "k", k.dtype)
    pv = _dev(v, "v", k.dtype, (B, H, T, dv))
    pa = _dev(log_decay, "log_decay", torch.float32, (B, H, T))
    if out is None:
        out = torch.empty((B, H, Lmax, dk, dv), dtype=torch.float32, device=k.device)
    po = _dev(out, "out", torch.float32, (B, H, Lmax, dk, dv))
    need = loglin_prefill_workspace_bytes(B, H, T, dk, dv, Lmax)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=k.device)
    pw = _dev(workspace, "workspace") if workspace is not None else None
    nws = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_load().loglin_prefill_states(pk, pv, pa, po, B, H, T, dk, dv, Lmax, _DTYPES[k.dtype],
                                         pw, nws, _stream(k)))
    return out


# ---------------------------------------------------------------- decode

@dataclass
class DecodeState:
    handle: ctypes.c_void_p
    nseq: int
    H: int
    dk: int
    dv: int
    Lmax: int
    device: torch.device

    def __del__(self):
        if self.handle and _lib is not None:
            try:
                _lib.loglin_state_free(self.handle)
            except Exception:
                pass
            self.handle = None


def loglin_state_init(nseq: int, H: int, dk: int, dv: int, Lmax: int, device=None) -> DecodeState:
    device = torch.device(device or "cuda")
    h = ctypes.c_void_p()
    s = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    _check(_load().loglin_state_init(ctypes.byref(h), nseq, H, dk, dv, Lmax, s))
    return DecodeState(h, nseq, H, dk, dv, Lmax, device)


def loglin_state_free(st: DecodeState) -> None:
    if st.handle:
        h, st.handle = st.handle, None
        _check(_load().loglin_state_free(h))


def loglin_state_load(st: DecodeState, pos, levels=None) -> None:
    """pos: next position per sequence (host ints); levels: [nseq,H,Lmax,dk,dv] float32 or None."""
    p = torch.as_tensor(pos, dtype=torch.int64).contiguous().cpu()
    if tuple(p.shape) != (st.nseq,):
        raise ValueError(f"pos must have shape ({st.nseq},)")
    pl = None
    if levels is not None:
        pl = _dev(levels, "levels", torch.float32, (st.nseq, st.H, st.Lmax, st.dk, st.dv))
    s = ctypes.c_void_p(torch.cuda.current_stream(st.device).cuda_stream)
    _check(_load().loglin_state_load(st.handle, p.data_ptr(), pl, s))


def loglin_state_export(st: DecodeState, levels: bool = True):
    """Returns (pos int64 host tensor, levels [nseq,H,Lmax,dk,dv] float32 or None)."""
    pos = torch.empty(st.nseq, dtype=torch.int64)
    lv = None
    if levels:
        lv = torch.empty((st.nseq, st.H, st.Lmax, st.dk, st.dv), dtype=torch.float32,
                         device=st.device)
    s = ctypes.c_void_p(torch.cuda.current_stream(st.device).cuda_stream)
    _check(_load().loglin_state_export(st.handle, pos.data_ptr(),
                                       lv.data_ptr() if lv is not None else None, s))
    return pos, lv


def loglin_decode_step(st: DecodeState, q, k, v, log_decay, lam, out=None):
    """One Fenwick step for every (sequence, head); returns out [nseq,H,dv] float32."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be float32 or bfloat16 (got {q.dtype})")
    pq = _dev(q, "q", q.dtype, (st.nseq, st.H, st.dk))
    pk = _dev(k, "k", q.dtype, (st.nseq, st.H, st.dk))
    pv = _dev(v, "v", q.dtype, (st.nseq, st.H, st.dv))
    pa = _dev(log_decay, "log_decay", torch.float32, (st.nseq, st.H))
    pl = _dev(lam, "lam", torch.float32, (st.nseq, st.H, st.Lmax))
    if out is None:
        out = torch.empty((st.nseq, st.H, st.dv), dtype=torch.float32, device=q.device)
    po = _dev(out, "out", torch.float32, (st.nseq, st.H, st.dv))
    _check(_load().loglin_decode_step(st.handle, pq, pk, pv, pa, pl, po, _DTYPES[q.dtype],
                                      _stream(q)))
    return out


def loglin_gdn_decode_step(st: DecodeState, q, k, v, log_decay, beta, lam, out=None):
    """One log-linear Gated DeltaNet decode step: q, k [nseq,H,dk], v [nseq,H,dv],
    log_decay and beta [nseq,H], lam [nseq,H,Lmax].  Returns out [nseq,H,dv]."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be float32 or bfloat16 (got {q.dtype})")
    pq = _dev(q, "q", q.dtype, (st.nseq, st.H, st.dk))
    pk = _dev(k, "k", q.dtype, (st.nseq, st.H, st.dk))
    pv = _dev(v, "v", q.dtype, (st.nseq, st.H, st.dv))
    pa = _dev(log_decay, "log_decay", torch.float32, (st.nseq, st.H))
    pb = _dev(beta, "beta", torch.float32, (st.nseq, st.H))
    pl = _dev(lam, "lam", torch.float32, (st.nseq, st.H, st.Lmax))
    if out is None:
        out = torch.empty((st.nseq, st.H, st.dv), dtype=torch.float32, device=q.device)
    po = _dev(out, "out", torch.float32, (st.nseq, st.H, st.dv))
    _check(_load().loglin_gdn_decode_step(st.handle, pq, pk, pv, pa, pb, pl, po, _DTYPES[q.dtype],
                                          _stream(q)))
    return out


def loglin_debug_level_map(T: int, device=None):
    device = torch.device(device or "cuda")
    out = torch.empty((T, T), dtype=torch.int8, device=device)
    s = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    _check(_load().loglin_debug_level_map(T, out.data_ptr(), s))
    return out
