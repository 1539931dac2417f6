"""Python binding of libattn.so (MI355X / gfx950 attention forward + backward).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI in ``include/attn.h``.  torch supplies device memory
and the current stream.  The binding fails loudly if the library is not built;
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libattn.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARGUMENT = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_WORKSPACE_TOO_SMALL = 3
ATTN_ERR_HIP = 4
ATTN_FP16 = 0
ATTN_BF16 = 1

EXPORTED_SYMBOLS = ("attn_fwd", "attn_bwd_workspace_size", "attn_bwd", "attn_bwd_phases", "attn_bwd_noalloc",
                    "attn_status_string", "attn_version")
NOALLOC_SCRATCH_BYTES = 32 << 20  # ATTN_NOALLOC_SCRATCH_BYTES in include/attn.h
PHASE_PREPROCESS = 1
PHASE_DKDV = 2
PHASE_DQ = 4
PHASE_ALL = 7


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


class attn_strides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("row", ctypes.c_int64), ("head", ctypes.c_int64)]


class attn_params(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("batch", ctypes.c_int32),
        ("seqlen_q", ctypes.c_int32),
        ("seqlen_k", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("deterministic", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("total_q", ctypes.c_int32),
        ("total_k", ctypes.c_int32),
        ("q", attn_strides),
        ("k", attn_strides),
        ("v", attn_strides),
        ("o", attn_strides),
        ("dout", attn_strides),
        ("dq", attn_strides),
        ("dk", attn_strides),
        ("dv", attn_strides),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} not found: build it with `python -m flashattention_backward_pass_attn_amd.build` "
            "(or __graft_entry__.build()); there is no CPU fallback")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(attn_params)
    vp = ctypes.c_void_p
    lib.attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_bwd_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.attn_bwd_workspace_size.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_phases.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp,
                                    ctypes.c_uint]
    lib.attn_bwd_phases.restype = ctypes.c_int
    lib.attn_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.attn_bwd_noalloc.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().attn_status_string(status).decode()


def _check(status: int, where: str):
    if status != ATTN_OK:
        raise AttnError(status, where, status_string(status))


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return ATTN_FP16
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"attention tensors must be float16 or bfloat16, got {t.dtype}")


def _strides(t, varlen: bool) -> attn_strides:
    if t.stride(-1) != 1:
        raise ValueError("last dimension must be contiguous")
    if varlen:  # [total, heads, dim]
        return attn_strides(0, t.stride(0), t.stride(1))
    return attn_strides(t.stride(0), t.stride(1), t.stride(2))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def make_params(q, k, causal: bool, softmax_scale: Optional[float] = None, deterministic: bool = False,
                cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q: Optional[int] = None,
                max_seqlen_k: Optional[int] = None, window=(-1, -1)) -> attn_params:
    """Fill attn_params from Q/K tensors.  Strides of the other tensors are set by the callers.

    ``window = (left, right)``: local attention (see attn_params in include/attn.h), -1 = no bound."""
    varlen = cu_seqlens_q is not None
    p = attn_params()
    p.dtype = _dtype_code(q)
    if varlen:
        if cu_seqlens_k is None or max_seqlen_q is None or max_seqlen_k is None:
            raise ValueError("varlen needs cu_seqlens_q, cu_seqlens_k, max_seqlen_q and max_seqlen_k")
        p.batch = cu_seqlens_q.numel() - 1
        p.seqlen_q, p.seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
        p.heads_q, p.heads_kv, p.head_dim = q.shape[1], k.shape[1], q.shape[2]
        p.cu_seqlens_q, p.cu_seqlens_k = cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr()
        p.total_q, p.total_k = q.shape[0], k.shape[0]
    else:
        p.batch, p.seqlen_q, p.heads_q, p.head_dim = q.shape
        p.seqlen_k, p.heads_kv = k.shape[1], k.shape[2]
    p.softmax_scale = (1.0 / math.sqrt(p.head_dim)) if softmax_scale is None else float(softmax_scale)
    p.causal = 1 if causal else 0
    p.deterministic = 1 if deterministic else 0
    p.window_left, p.window_right = int(window[0]), int(window[1])
    return p


def _stream_ptr(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _check_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def attn_fwd(q, k, v, causal: bool = False, softmax_scale: Optional[float] = None, cu_seqlens_q=None,
             cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, out=None, lse=None, window=(-1, -1)):
    """O, LSE = attention forward.  Layout [b, s, h, d] (varlen [total, h, d]).

    LSE is fp32 natural log, [b, h, Sq] (varlen [h, total_q]).
    """
    torch = _torch()
    lib = load_library()
    _check_device(q, k, v)
    varlen = cu_seqlens_q is not None
    p = make_params(q, k, causal, softmax_scale, False, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    window)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        shape = (q.shape[1], q.shape[0]) if varlen else (q.shape[0], q.shape[2], q.shape[1])
        lse = torch.empty(shape, dtype=torch.float32, device=q.device)
    p.q, p.k, p.v, p.o = (_strides(t, varlen) for t in (q, k, v, out))
    st = lib.attn_fwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      _stream_ptr(q.device))
    _check(st, "attn_fwd")
    return out, lse


def bwd_workspace_size(p: attn_params) -> int:
    """Workspace bytes attn_bwd needs: Delta and LSE*log2(e), fp32, O(Sq) per head."""
    n = ctypes.c_size_t(0)
    lib = load_library()
    _check(lib.attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)), "attn_bwd_workspace_size")
    return n.value


def attn_bwd(q, k, v, o, lse, dout, causal: bool = False, softmax_scale: Optional[float] = None,
             deterministic: bool = False, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
             max_seqlen_k=None, dq=None, dk=None, dv=None, workspace=None, return_delta: bool = False,
             phases: int = PHASE_ALL, window=(-1, -1)):
    """dQ, dK, dV (and optionally Delta) of sum(O * dO) for attention.

    ``phases`` selects the kernels to launch: the dQ kernel (which also runs
    the preprocess for its rows), the dK/dV kernel, and the standalone
    preprocess, which runs only without the dQ phase (see attn_bwd_phases in
    include/attn.h); the default launches dQ, then dK/dV.  Without a
    ``workspace`` one of ``bwd_workspace_size()`` bytes is allocated (two fp32
    row statistics per query row and head).
    """
    torch = _torch()
    lib = load_library()
    _check_device(q, k, v, o, lse, dout)
    varlen = cu_seqlens_q is not None
    p = make_params(q, k, causal, softmax_scale, deterministic, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                    max_seqlen_k, window)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        setattr(p, name, _strides(t, varlen))
    need = bwd_workspace_size(p)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    delta = torch.empty_like(lse) if return_delta else None
    args = (ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _ptr(delta), _stream_ptr(q.device))
    if phases == PHASE_ALL:
        st = lib.attn_bwd(*args)
    else:
        st = lib.attn_bwd_phases(*args, phases)
    _check(st, "attn_bwd")
    if return_delta:
        return dq, dk, dv, delta
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, dout, causal: bool = False, softmax_scale: Optional[float] = None,
                     deterministic: bool = False, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
                     max_seqlen_k=None, dq=None, dk=None, dv=None, return_delta: bool = False, window=(-1, -1)):
    """attn_bwd through the entry point that allocates nothing on the device:
    its statistics live in the library's static scratch array (see
    attn_bwd_noalloc in include/attn.h).  The outputs are allocated here only
    when not given."""
    torch = _torch()
    lib = load_library()
    _check_device(q, k, v, o, lse, dout)
    varlen = cu_seqlens_q is not None
    p = make_params(q, k, causal, softmax_scale, deterministic, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                    max_seqlen_k, window)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        setattr(p, name, _strides(t, varlen))
    delta = torch.empty_like(lse) if return_delta else None
    st = lib.attn_bwd_noalloc(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                              _ptr(delta), _stream_ptr(q.device))
    _check(st, "attn_bwd_noalloc")
    if return_delta:
        return dq, dk, dv, delta
    return dq, dk, dv


def version() -> str:
    return load_library().attn_version().decode()
