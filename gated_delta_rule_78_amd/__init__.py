"""MI355X (gfx950) Kimi Delta Attention (KDA) hot path: Python binding of ``libkda.so``.

The binding only marshals arguments: it allocates outputs and workspace with torch (device
memory and streams) and passes raw device pointers to the C ABI declared in ``include/kda.h``.
Every step of the computation runs in the library's HIP kernels. There is no fallback: if the
library is missing or fails, the call raises.

    chunk_fwd(q, k, v, log_alpha, beta, S0=None) -> (o, S_T)     chunkwise prefill
    chunk_fwd_noalloc(q, k, v, log_alpha, beta, S0=None)          the same, workspace from the
        -> (o, S_T)                                               library's fixed scratch
    chunk_fwd_varlen(q, k, v, log_alpha, beta, cu_seqlens, ...)   packed variable-length batch,
        -> (o, S_T, S_ckpt, ckpt_offsets)                         state checkpoints every E tokens
    chunk_bwd(q, k, v, log_alpha, beta, S0, dO, dS_T) -> grads    backward of chunkwise prefill
    decode_step(q, k, v, log_alpha, beta, S) -> o                 one token, S updated in place
"""
import contextlib
import ctypes
import os

import torch

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "SCRATCH_BYTES", "chunk_fwd_varlen", "chunk_bwd", "chunk_bwd_workspace_bytes", "decode_step", "chunk_workspace_bytes", "varlen_workspace_bytes",
           "library", "KDAError", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
_DTYPES = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}


class ChunkDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64), ("dk", ctypes.c_int64),
                ("dv", ctypes.c_int64), ("chunk", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("segments", ctypes.c_int32), ("state_pass", ctypes.c_int32)]


# kda_chunk_desc::state_pass
STATE_PASS_AUTO, STATE_PASS_TWO_KERNELS, STATE_PASS_FUSED = 0, 1, 2


class VarlenDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64), ("max_len", ctypes.c_int64),
                ("dk", ctypes.c_int64), ("dv", ctypes.c_int64), ("chunk", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("segments", ctypes.c_int32), ("ckpt_every", ctypes.c_int32),
                ("packed", ctypes.c_int32), ("state_pass", ctypes.c_int32)]


class Gating(ctypes.Structure):
    _fields_ = [("z", ctypes.c_void_p), ("A_log", ctypes.c_void_p), ("g_min", ctypes.c_float), ("eps", ctypes.c_float),
                ("gate", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p)]


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
        lib.kda_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(ChunkDesc), P, P, P, P, P, P, P, P, P]
        lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int32
        lib.kda_chunk_fwd_varlen_workspace_bytes.argtypes = [ctypes.POINTER(VarlenDesc)]
        lib.kda_chunk_fwd_varlen_workspace_bytes.restype = ctypes.c_size_t
        lib.kda_chunk_fwd_varlen.argtypes = [ctypes.POINTER(VarlenDesc), P, P, P, P, P, P, P, P, P, P, P,
                                             ctypes.POINTER(Gating), P, ctypes.c_size_t, P]
        lib.kda_chunk_fwd_varlen.restype = ctypes.c_int32
        lib.kda_chunk_bwd_workspace_bytes.argtypes = [ctypes.POINTER(ChunkDesc)]
        lib.kda_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.kda_chunk_bwd.argtypes = [ctypes.POINTER(ChunkDesc)] + [P] * 15 + [ctypes.c_size_t, P]
        lib.kda_chunk_bwd.restype = ctypes.c_int32
        lib.kda_decode_step.argtypes = [ctypes.POINTER(DecodeDesc), P, P, P, P, P, P, P, P]
        lib.kda_decode_step.restype = ctypes.c_int32
        lib.kda_decode_step_gated.argtypes = [ctypes.POINTER(DecodeDesc), P, P, P, P, P, ctypes.POINTER(Gating), P, P,
                                              P]
        lib.kda_decode_step_gated.restype = ctypes.c_int32
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


def _alloc_on(stream):
    """Context in which the binding allocates outputs and workspace: the caller's ``stream`` when
    one is given, so that the caching allocator ties those blocks to the stream the kernels run
    on (a block freed on return is then reused only behind them), else a no-op."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _check_device(fn, dev):
    if dev.type != "cuda":
        raise ValueError("%s runs on the GPU; got a tensor on %s" % (fn, dev))


def _check_workspace(workspace, dev):
    """A caller's workspace must be a contiguous tensor on ``dev``: a wrong device or a strided view
    is a ValueError here, not an out-of-range access in the kernels."""
    if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on %s (got %s, contiguous=%s)"
                         % (dev, workspace.device, workspace.is_contiguous()))


def _workspace(need, workspace, dev):
    """The caller's (checked) workspace when it holds ``need`` bytes, else a new one."""
    if workspace is not None and workspace.numel() * workspace.element_size() >= need:
        return workspace
    return torch.empty(need, device=dev, dtype=torch.uint8) if need else workspace


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _check(fn, status):
    if status != 0:
        raise KDAError(fn, status, library().kda_status_string(status).decode())


def _chunk_desc(q, v, segments, out_dtype, state_pass=STATE_PASS_AUTO):
    B, H, T, dk = q.shape
    return ChunkDesc(B, H, T, dk, v.shape[-1], 64, _DTYPES[q.dtype], _DTYPES[out_dtype], int(segments),
                     int(state_pass))


def chunk_workspace_bytes(q, v, segments=0, out_dtype=None, state_pass=STATE_PASS_AUTO):
    d = _chunk_desc(q, v, segments, out_dtype or q.dtype, state_pass)
    return int(library().kda_chunk_fwd_workspace_bytes(ctypes.byref(d)))


def _check_tensor(name, t, device, dtype, shape):
    if t.device != device or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s on %s (got %s %s %s)"
                         % (name, dtype, tuple(shape), device, t.dtype, tuple(t.shape), t.device))


def chunk_fwd(q, k, v, log_alpha, beta, S0=None, *, out_dtype=None, segments=0, state_pass=STATE_PASS_AUTO, o=None,
              S_T=None, store_state=True, workspace=None, stream=None):
    """Chunkwise KDA prefill through ``kda_chunk_fwd``.

    q, k, log_alpha: [B,H,T,dk]; v: [B,H,T,dv]; beta: [B,H,T] (all bf16 or all fp32);
    S0: [B,H,dk,dv] fp32 or None. Returns (o [B,H,T,dv], S_T [B,H,dk,dv] fp32 or None).
    ``segments`` and ``state_pass`` are kda_chunk_desc's (0: the library's choice).
    Caller-supplied o, S_T (may be S0) and workspace are checked like the inputs. Outputs and
    workspace the binding allocates are allocated on ``stream`` (default: the current stream).
    """
    dev = q.device
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("unsupported input dtype %s" % dt)
    out_dtype = out_dtype or dt
    if out_dtype not in _DTYPES:
        raise ValueError("unsupported output dtype %s" % out_dtype)
    for name, t, shape in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("log_alpha", log_alpha, (B, H, T, dk)),
                           ("v", v, (B, H, T, dv)), ("beta", beta, (B, H, T))):
        _check_tensor(name, t, dev, dt, shape)
    if S0 is not None:
        _check_tensor("S0", S0, dev, torch.float32, (B, H, dk, dv))
    if o is not None:
        _check_tensor("o", o, dev, out_dtype, (B, H, T, dv))
    if S_T is not None:
        _check_tensor("S_T", S_T, dev, torch.float32, (B, H, dk, dv))
    _check_workspace(workspace, dev)
    _check_device("chunk_fwd", dev)
    desc = _chunk_desc(q, v, segments, out_dtype, state_pass)
    lib = library()
    need = int(lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(desc)))
    with _alloc_on(stream):
        if o is None:
            o = torch.empty(B, H, T, dv, device=dev, dtype=out_dtype)
        if S_T is None and store_state:
            S_T = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32)
        workspace = _workspace(need, workspace, dev)
        st = lib.kda_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0),
                               _ptr(o), _ptr(S_T), _ptr(workspace), _nbytes(workspace), _stream(dev, stream))
    _check("kda_chunk_fwd", st)
    return o, S_T


def chunk_fwd_noalloc(q, k, v, log_alpha, beta, S0=None, *, out_dtype=None, o=None, S_T=None, store_state=True,
                      stream=None):
    """``chunk_fwd`` through ``kda_chunk_fwd_noalloc``: the library takes the workspace from its own
    fixed scratch (``SCRATCH_BYTES`` per device) instead of an argument, so the C call allocates
    nothing; pass ``o`` (and ``S_T``) to keep the binding from allocating them. Calls that overlap
    in time on one device share that scratch and race. Raises KDAError (KDA_ERR_SCRATCH) when the
    call needs more workspace than the scratch holds."""
    dev = q.device
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("unsupported input dtype %s" % dt)
    out_dtype = out_dtype or dt
    if out_dtype not in _DTYPES:
        raise ValueError("unsupported output dtype %s" % out_dtype)
    for name, t, shape in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("log_alpha", log_alpha, (B, H, T, dk)),
                           ("v", v, (B, H, T, dv)), ("beta", beta, (B, H, T))):
        _check_tensor(name, t, dev, dt, shape)
    if S0 is not None:
        _check_tensor("S0", S0, dev, torch.float32, (B, H, dk, dv))
    if o is not None:
        _check_tensor("o", o, dev, out_dtype, (B, H, T, dv))
    if S_T is not None:
        _check_tensor("S_T", S_T, dev, torch.float32, (B, H, dk, dv))
    _check_device("chunk_fwd_noalloc", dev)
    desc = _chunk_desc(q, v, 0, out_dtype)
    with _alloc_on(stream):
        if o is None:
            o = torch.empty(B, H, T, dv, device=dev, dtype=out_dtype)
        if S_T is None and store_state:
            S_T = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32)
        st = library().kda_chunk_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                             _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T), _stream(dev, stream))
    _check("kda_chunk_fwd_noalloc", st)
    return o, S_T


SCRATCH_BYTES = 192 << 20   # KDA_NOALLOC_SCRATCH_BYTES of include/kda.h


def _gating(dev, H, dv, dtype, lead, z, A_log, g_min, gate, norm_weight, eps):
    """kda_gating for the fused prologue (z, A_log, g_min) and epilogue (gate, norm_weight, eps),
    or None when neither is asked for."""
    if z is None and gate is None:
        return None
    if z is not None:
        _check_tensor("z", z, dev, dtype, z.shape)
        if tuple(z.shape[:-1]) != tuple(lead):
            raise ValueError("z must have the shape of log_alpha")
        _check_tensor("A_log", A_log, dev, torch.float32, (H,))
    if gate is not None:
        _check_tensor("gate", gate, dev, dtype, tuple(lead) + (dv,))
        if norm_weight is not None:
            _check_tensor("norm_weight", norm_weight, dev, torch.float32, (dv,))
    return Gating(_ptr(z), _ptr(A_log) if z is not None else None, float(g_min), float(eps), _ptr(gate),
                  _ptr(norm_weight) if gate is not None else None)


def _varlen_desc(N, H, T, max_len, dk, dv, out_dtype, segments, ckpt_every, packed, state_pass=STATE_PASS_AUTO):
    return VarlenDesc(N, H, T, max_len, dk, dv, 64, KDA_BF16, _DTYPES[out_dtype], int(segments), int(ckpt_every),
                      int(packed), int(state_pass))


def varlen_workspace_bytes(N, H, T, max_len, dk, dv, *, segments=0, ckpt_every=0, packed=True,
                           out_dtype=torch.bfloat16, state_pass=STATE_PASS_AUTO):
    d = _varlen_desc(N, H, T, max_len, dk, dv, out_dtype, segments, ckpt_every, packed, state_pass)
    return int(library().kda_chunk_fwd_varlen_workspace_bytes(ctypes.byref(d)))


def chunk_fwd_varlen(q, k, v, log_alpha, beta, cu_seqlens=None, S0=None, *, max_len=None, N=None, ckpt_every=0,
                     out_dtype=None, segments=0, state_pass=STATE_PASS_AUTO, o=None, S_T=None, S_ckpt=None,
                     ckpt_offsets=None, z=None, A_log=None, g_min=-5.0, gate=None, norm_weight=None, eps=1e-6,
                     store_state=True, workspace=None, stream=None):
    """KDA prefill over a batch of sequences with state checkpoints, through ``kda_chunk_fwd_varlen``.

    Packed (``cu_seqlens`` given, int32 [N+1] on the device): q, k, log_alpha [H,T,dk], v [H,T,dv],
    beta [H,T], bf16; sequence s is rows cu_seqlens[s]:cu_seqlens[s+1] of every head.
    ``max_len`` bounds every length (default T); ``N`` defaults to len(cu_seqlens) - 1.
    Equal lengths (``cu_seqlens`` None): tensors [N,H,T,...] as ``chunk_fwd``.
    S0, S_T: [N,H,dk,dv] fp32. With ``ckpt_every`` = E > 0, the state after every E tokens of each
    sequence goes to S_ckpt[ckpt_offsets[s] + j - 1, h] (S_ckpt: [K, H, dk, dv] fp32 with
    K >= T // E packed or N * (T // E) otherwise) and ckpt_offsets (int32 [N+1]) is written.
    Returns (o, S_T, S_ckpt, ckpt_offsets); the last two are None when E = 0. S_ckpt is returned
    at its capacity T // E (packed) or N * (T // E); its first ckpt_offsets[N] entries are written
    (the count is only known on the device, and reading it would synchronise).
    Fused prologue: with ``z`` (shape of log_alpha, which may then be None) and ``A_log`` [H] fp32,
    the log decay is g_min * sigmoid(exp(A_log[h]) * z). Fused epilogue: with ``gate`` (shape of
    v), o receives sigmoid(gate) * norm_weight * o / sqrt(mean(o^2) + eps).
    ``segments`` and ``state_pass`` are kda_varlen_desc's (0: the library's choice).
    Caller-supplied outputs and workspace are checked like the inputs; the ones the binding
    allocates are allocated on ``stream``.
    """
    dev = q.device
    if q.dtype != torch.bfloat16:
        raise ValueError("chunk_fwd_varlen takes bf16 inputs (got %s)" % q.dtype)
    out_dtype = out_dtype or q.dtype
    if out_dtype not in _DTYPES:
        raise ValueError("unsupported output dtype %s" % out_dtype)
    packed = cu_seqlens is not None
    dk, dv = q.shape[-1], v.shape[-1]
    if packed:
        H, T = q.shape[0], q.shape[1]
        _check_tensor("cu_seqlens", cu_seqlens, dev, torch.int32, (cu_seqlens.numel(),))
        N = cu_seqlens.numel() - 1 if N is None else N
        if N < 1 or cu_seqlens.numel() != N + 1:
            raise ValueError("cu_seqlens must have N + 1 >= 2 entries")
        lead, slead = (H, T), (N, H)
        max_len = T if max_len is None else int(max_len)
        n_ck = T // ckpt_every if ckpt_every else 0
    else:
        N, H, T = q.shape[0], q.shape[1], q.shape[2]
        lead, slead = (N, H, T), (N, H)
        max_len = T
        n_ck = N * (T // ckpt_every) if ckpt_every else 0
    for name, t, shape in (("q", q, lead + (dk,)), ("k", k, lead + (dk,)), ("log_alpha", log_alpha, lead + (dk,)),
                           ("v", v, lead + (dv,)), ("beta", beta, lead)):
        if t is None and name == "log_alpha" and z is not None:
            continue
        _check_tensor(name, t, dev, torch.bfloat16, shape)
    gating = _gating(dev, H, dv, torch.bfloat16, lead, z, A_log, g_min, gate, norm_weight, eps)
    if S0 is not None:
        _check_tensor("S0", S0, dev, torch.float32, slead + (dk, dv))
    if o is not None:
        _check_tensor("o", o, dev, out_dtype, lead + (dv,))
    if S_T is not None:
        _check_tensor("S_T", S_T, dev, torch.float32, slead + (dk, dv))
    if ckpt_every:
        if S_ckpt is not None:
            if (S_ckpt.device != dev or S_ckpt.dtype != torch.float32 or not S_ckpt.is_contiguous()
                    or S_ckpt.dim() != 4 or tuple(S_ckpt.shape[1:]) != (H, dk, dv) or S_ckpt.shape[0] < n_ck):
                raise ValueError("S_ckpt must be a contiguous float32 tensor [K, %d, %d, %d] with K >= %d on %s "
                                 "(got %s %s %s)" % (H, dk, dv, n_ck, dev, S_ckpt.dtype, tuple(S_ckpt.shape),
                                                     S_ckpt.device))
        if ckpt_offsets is not None:
            _check_tensor("ckpt_offsets", ckpt_offsets, dev, torch.int32, (N + 1,))
    _check_workspace(workspace, dev)
    _check_device("chunk_fwd_varlen", dev)
    desc = _varlen_desc(N, H, T, max_len, dk, dv, out_dtype, segments, ckpt_every, packed, state_pass)
    lib = library()
    need = int(lib.kda_chunk_fwd_varlen_workspace_bytes(ctypes.byref(desc)))
    with _alloc_on(stream):
        if o is None:
            o = torch.empty(lead + (dv,), device=dev, dtype=out_dtype)
        if S_T is None and store_state:
            S_T = torch.empty(slead + (dk, dv), device=dev, dtype=torch.float32)
        if ckpt_every:
            if S_ckpt is None:
                S_ckpt = torch.empty(max(n_ck, 1), H, dk, dv, device=dev, dtype=torch.float32)
            if ckpt_offsets is None:
                ckpt_offsets = torch.empty(N + 1, device=dev, dtype=torch.int32)
        workspace = _workspace(need, workspace, dev)
        st = lib.kda_chunk_fwd_varlen(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                      _ptr(cu_seqlens), _ptr(S0), _ptr(o), _ptr(S_T),
                                      _ptr(S_ckpt if ckpt_every else None), _ptr(ckpt_offsets if ckpt_every else None),
                                      None if gating is None else ctypes.byref(gating),
                                      _ptr(workspace), _nbytes(workspace), _stream(dev, stream))
    _check("kda_chunk_fwd_varlen", st)
    if not ckpt_every:
        return o, S_T, None, None
    return o, S_T, S_ckpt[:n_ck], ckpt_offsets


def chunk_bwd_workspace_bytes(q, v, segments=0, out_dtype=None):
    d = _chunk_desc(q, v, segments, out_dtype or q.dtype)
    return int(library().kda_chunk_bwd_workspace_bytes(ctypes.byref(d)))


def chunk_bwd(q, k, v, log_alpha, beta, S0, dO, dS_T=None, *, segments=0, workspace=None, stream=None):
    """Backward of chunkwise prefill through ``kda_chunk_bwd`` (bf16 inputs).

    Inputs as ``chunk_fwd``; dO [B,H,T,dv] (bf16 or fp32: the forward's output type), dS_T
    [B,H,dk,dv] fp32 or None. Returns fp32 (dq, dk, dv, dlog_alpha, dbeta, dS0), allocated on
    ``stream``."""
    dev = q.device
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if q.dtype != torch.bfloat16:
        raise ValueError("chunk_bwd takes bf16 inputs (got %s)" % q.dtype)
    for name, t, shape in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("log_alpha", log_alpha, (B, H, T, dk)),
                           ("v", v, (B, H, T, dv)), ("beta", beta, (B, H, T))):
        _check_tensor(name, t, dev, torch.bfloat16, shape)
    if S0 is not None:
        _check_tensor("S0", S0, dev, torch.float32, (B, H, dk, dv))
    if dO.dtype not in _DTYPES:
        raise ValueError("unsupported dO dtype %s" % dO.dtype)
    _check_tensor("dO", dO, dev, dO.dtype, (B, H, T, dv))
    if dS_T is not None:
        _check_tensor("dS_T", dS_T, dev, torch.float32, (B, H, dk, dv))
    _check_workspace(workspace, dev)
    _check_device("chunk_bwd", dev)
    desc = _chunk_desc(q, v, segments, dO.dtype)
    lib = library()
    need = int(lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(desc)))
    f32 = dict(device=dev, dtype=torch.float32)
    with _alloc_on(stream):
        dq, dk_, dla = (torch.empty(B, H, T, dk, **f32) for _ in range(3))
        dv_ = torch.empty(B, H, T, dv, **f32)
        dbeta = torch.empty(B, H, T, **f32)
        dS0 = torch.empty(B, H, dk, dv, **f32)
        workspace = _workspace(need, workspace, dev)
        st = lib.kda_chunk_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0),
                               _ptr(dO), _ptr(dS_T), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dla), _ptr(dbeta), _ptr(dS0),
                               _ptr(workspace), _nbytes(workspace), _stream(dev, stream))
    _check("kda_chunk_bwd", st)
    return dq, dk_, dv_, dla, dbeta, dS0


def decode_step(q, k, v, log_alpha, beta, S, *, out_dtype=None, o=None, z=None, A_log=None, g_min=-5.0, gate=None,
                norm_weight=None, eps=1e-6, stream=None):
    """One KDA decode step through ``kda_decode_step``; S ([N,H,dk,dv] fp32) is updated in place.

    q, k, log_alpha: [N,H,dk]; v: [N,H,dv]; beta: [N,H]. Returns o [N,H,dv] (allocated on ``stream``
    when not given). With ``z`` or ``gate``, the fused prologue / epilogue of ``chunk_fwd_varlen``
    (``kda_decode_step_gated``)."""
    dev = q.device
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("unsupported input dtype %s" % dt)
    out_dtype = out_dtype or dt
    if out_dtype not in _DTYPES:
        raise ValueError("unsupported output dtype %s" % out_dtype)
    for name, t, shape in (("q", q, (N, H, dk)), ("k", k, (N, H, dk)), ("log_alpha", log_alpha, (N, H, dk)),
                           ("v", v, (N, H, dv)), ("beta", beta, (N, H))):
        if t is None and name == "log_alpha" and z is not None:
            continue
        _check_tensor(name, t, dev, dt, shape)
    gating = _gating(dev, H, dv, dt, (N, H), z, A_log, g_min, gate, norm_weight, eps)
    _check_tensor("S", S, dev, torch.float32, (N, H, dk, dv))
    if o is not None:
        _check_tensor("o", o, dev, out_dtype, (N, H, dv))
    _check_device("decode_step", dev)
    desc = DecodeDesc(N, H, dk, dv, _DTYPES[dt], _DTYPES[out_dtype])
    with _alloc_on(stream):
        if o is None:
            o = torch.empty(N, H, dv, device=dev, dtype=out_dtype)
        if gating is None:
            st = library().kda_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                           _ptr(S), _ptr(o), _stream(dev, stream))
            fn = "kda_decode_step"
        else:
            st = library().kda_decode_step_gated(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                                 _ptr(beta), ctypes.byref(gating), _ptr(S), _ptr(o),
                                                 _stream(dev, stream))
            fn = "kda_decode_step_gated"
    _check(fn, st)
    return o
