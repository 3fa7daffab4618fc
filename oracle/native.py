"""Build and call the plain C fp64 oracle (``kda_oracle.c``). Test infrastructure only.

The recurrence it implements is the state equation of section 2.2 of the Kimi K3 reading notes
(liuzhao09.github.io/papers/kimi-k3.html): decay each key-channel row by alpha_t, write
beta_t k_t (v_t - S^T k_t)^T, then read o_t = S_t^T q_t.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ``kda_oracle.c`` with gcc (fp64, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.kda_oracle_fwd.argtypes = [I64, I64, I64, I64, P, P, P, P, P, P, P, I64, P, P, I64, P, ctypes.c_int]
        lib.kda_oracle_fwd.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


def kda_fwd(q, k, v, log_alpha, beta, S0=None, rows=None, threads=None, want_o=True, ckpt_every=0):
    """Token-by-token fp64 KDA over lanes.

    q, k, log_alpha: [L, T, dk]; v: [L, T, dv]; beta: [L, T]; S0: [L, dk, dv] or None.
    Every value must be exactly representable in fp32 (bf16 and fp32 inputs are).
    rows: optional sorted token indices whose outputs are kept.
    Returns (o [L, len(rows) or T, dv] float64 or None, S_T [L, dk, dv] float64), and with
    ckpt_every = E > 0 a third array [L, T // E, dk, dv]: the state after the first j*E tokens.
    """
    lib = _load()
    q, k, v, la, beta, S0 = (_f32(a) for a in (q, k, v, log_alpha, beta, S0))
    L, T, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (L, T, dk) and la.shape == (L, T, dk) and v.shape == (L, T, dv)
    assert beta.shape == (L, T)
    if S0 is not None:
        assert S0.shape == (L, dk, dv)
    r = None
    if rows is not None:
        r = np.ascontiguousarray(rows, dtype=np.int64)
    nrows = T if r is None else len(r)
    o = np.empty((L, nrows, dv), dtype=np.float64) if want_o else None
    ST = np.empty((L, dk, dv), dtype=np.float64)
    ck = np.empty((L, T // ckpt_every, dk, dv), dtype=np.float64) if ckpt_every else None
    rc = lib.kda_oracle_fwd(L, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(beta), _ptr(S0),
                            _ptr(r), 0 if r is None else len(r), _ptr(o), _ptr(ST),
                            int(ckpt_every), _ptr(ck), threads or default_threads())
    if rc != 0:
        raise ValueError("kda_oracle_fwd rejected its arguments")
    return (o, ST, ck) if ckpt_every else (o, ST)


def kda_varlen(q, k, v, log_alpha, beta, cu_seqlens, S0=None, ckpt_every=0, threads=None):
    """Packed batch of variable-length sequences: each (sequence s, head h) pair is an
    independent lane over rows cu_seqlens[s] .. cu_seqlens[s+1]-1 of head h.

    q, k, log_alpha: [H, T, dk]; v: [H, T, dv]; beta: [H, T]; S0: [N, H, dk, dv] or None.
    Returns (o [H, T, dv], S_T [N, H, dk, dv]) and, with ckpt_every = E > 0, the checkpoints
    [sum_s floor(len_s / E), H, dk, dv] (sequence-major, the states after every E tokens of each
    sequence) and their offsets [N + 1]."""
    cu = [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    H, T, dk = np.shape(q)
    dv = np.shape(v)[2]
    o = np.zeros((H, T, dv))
    ST = np.zeros((N, H, dk, dv))
    cks, offs = [], [0]
    for s in range(N):
        a, b = cu[s], cu[s + 1]
        s0 = None if S0 is None else np.asarray(S0)[s]
        res = kda_fwd(np.asarray(q)[:, a:b], np.asarray(k)[:, a:b], np.asarray(v)[:, a:b],
                      np.asarray(log_alpha)[:, a:b], np.asarray(beta)[:, a:b], s0, threads=threads,
                      ckpt_every=ckpt_every)
        o[:, a:b] = res[0]
        ST[s] = res[1]
        if ckpt_every:
            cks.append(np.transpose(res[2], (1, 0, 2, 3)))   # [n_s, H, dk, dv]
            offs.append(offs[-1] + res[2].shape[1])
    if not ckpt_every:
        return o, ST
    ck = np.concatenate(cks, axis=0) if cks else np.zeros((0, H, dk, dv))
    return o, ST, ck, np.array(offs, dtype=np.int64)


def kda_decode(q, k, v, log_alpha, beta, S):
    """One decode step = one iteration of the recurrence. q,k,log_alpha [L,dk]; v [L,dv];
    beta [L]; S [L,dk,dv]. Returns (o [L,dv], S' [L,dk,dv]) in float64."""
    q, k, v, la = (np.asarray(a)[:, None, :] for a in (q, k, v, log_alpha))
    o, S1 = kda_fwd(q, k, v, la, np.asarray(beta)[:, None], S0=S)
    return o[:, 0, :], S1
