"""MI355X (gfx950) Kimi Delta Attention (KDA) hot path: Python binding of ``libkda.so``.

The binding only marshals arguments: it allocates outputs and workspace with torch (device
memory and streams) and passes raw device pointers to the C ABI declared in ``include/kda.h``.
Every step of the computation runs in the library's HIP kernels. There is no fallback: if the
library is missing or fails, the call raises.

    chunk_fwd(q, k, v, log_alpha, beta, S0=None) -> (o, S_T)     chunkwise prefill
    decode_step(q, k, v, log_alpha, beta, S) -> o                 one token, S updated in place
"""
import ctypes
import os

import torch

__all__ = ["chunk_fwd", "decode_step", "chunk_workspace_bytes", "library", "KDAError", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
_DTYPES = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}


class ChunkDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64), ("dk", ctypes.c_int64),
                ("dv", ctypes.c_int64), ("chunk", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("segments", ctypes.c_int32)]


class DecodeDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("H", ctypes.c_int64), ("dk", ctypes.c_int64), ("dv", ctypes.c_int64),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


class KDAError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s" % (fn, msg))
        self.status = status


_lib = None


def library():
    """Load ``libkda.so`` (built by ``gated_delta_rule_78_amd.build``); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkda.so not found at %s: build it with "
                               "`python -m gated_delta_rule_78_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        lib.kda_chunk_fwd_workspace_bytes.argtypes = [ctypes.POINTER(ChunkDesc)]
        lib.kda_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.kda_chunk_fwd.argtypes = [ctypes.POINTER(ChunkDesc), P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.kda_chunk_fwd.restype = ctypes.c_int32
        lib.kda_decode_step.argtypes = [ctypes.POINTER(DecodeDesc), P, P, P, P, P, P, P, P]
        lib.kda_decode_step.restype = ctypes.c_int32
        lib.kda_status_string.argtypes = [ctypes.c_int32]
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_version.argtypes = []
        lib.kda_version.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != 0:
        raise KDAError(fn, status, library().kda_status_string(status).decode())


def _chunk_desc(q, v, segments, out_dtype):
    B, H, T, dk = q.shape
    return ChunkDesc(B, H, T, dk, v.shape[-1], 64, _DTYPES[q.dtype], _DTYPES[out_dtype], int(segments))


def chunk_workspace_bytes(q, v, segments=0, out_dtype=None):
    d = _chunk_desc(q, v, segments, out_dtype or q.dtype)
    return int(library().kda_chunk_fwd_workspace_bytes(ctypes.byref(d)))


def _check_tensor(name, t, device, dtype, shape):
    if t.device != device or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s on %s (got %s %s %s)"
                         % (name, dtype, tuple(shape), device, t.dtype, tuple(t.shape), t.device))


def chunk_fwd(q, k, v, log_alpha, beta, S0=None, *, out_dtype=None, segments=0, o=None, S_T=None,
              store_state=True, workspace=None, stream=None):
    """Chunkwise KDA prefill through ``kda_chunk_fwd``.

    q, k, log_alpha: [B,H,T,dk]; v: [B,H,T,dv]; beta: [B,H,T] (all bf16 or all fp32);
    S0: [B,H,dk,dv] fp32 or None. Returns (o [B,H,T,dv], S_T [B,H,dk,dv] fp32 or None).
    """
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_fwd runs on the GPU; got a tensor on %s" % dev)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("unsupported input dtype %s" % dt)
    out_dtype = out_dtype or dt
    for name, t, shape in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("log_alpha", log_alpha, (B, H, T, dk)),
                           ("v", v, (B, H, T, dv)), ("beta", beta, (B, H, T))):
        _check_tensor(name, t, dev, dt, shape)
    if S0 is not None:
        _check_tensor("S0", S0, dev, torch.float32, (B, H, dk, dv))
    if o is None:
        o = torch.empty(B, H, T, dv, device=dev, dtype=out_dtype)
    else:
        _check_tensor("o", o, dev, out_dtype, (B, H, T, dv))
    if S_T is None and store_state:
        S_T = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32)
    desc = _chunk_desc(q, v, segments, out_dtype)
    lib = library()
    need = int(lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(desc)))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.kda_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0),
                           _ptr(o), _ptr(S_T), _ptr(workspace), ws_bytes, _stream(dev, stream))
    _check("kda_chunk_fwd", st)
    return o, S_T


def decode_step(q, k, v, log_alpha, beta, S, *, out_dtype=None, o=None, stream=None):
    """One KDA decode step through ``kda_decode_step``; S ([N,H,dk,dv] fp32) is updated in place.

    q, k, log_alpha: [N,H,dk]; v: [N,H,dv]; beta: [N,H]. Returns o [N,H,dv]."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("decode_step runs on the GPU; got a tensor on %s" % dev)
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("unsupported input dtype %s" % dt)
    out_dtype = out_dtype or dt
    for name, t, shape in (("q", q, (N, H, dk)), ("k", k, (N, H, dk)), ("log_alpha", log_alpha, (N, H, dk)),
                           ("v", v, (N, H, dv)), ("beta", beta, (N, H))):
        _check_tensor(name, t, dev, dt, shape)
    _check_tensor("S", S, dev, torch.float32, (N, H, dk, dv))
    if o is None:
        o = torch.empty(N, H, dv, device=dev, dtype=out_dtype)
    else:
        _check_tensor("o", o, dev, out_dtype, (N, H, dv))
    desc = DecodeDesc(N, H, dk, dv, _DTYPES[dt], _DTYPES[out_dtype])
    st = library().kda_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                   _ptr(S), _ptr(o), _stream(dev, stream))
    _check("kda_decode_step", st)
    return o
