"""Shared helpers for the GPU parity tests: run the oracle on host copies of the exact device
inputs and compare with the tolerances of the KDA hot path:
  outputs      max-abs <= 2e-2 for bf16 inputs, <= 1e-4 for the fp32 path
  final state  relative L2 per lane (max over lanes) <= 1e-2 (fp32 path: 1e-4)."""
import sys

import numpy as np
import torch

from oracle import native

TOL_O = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
TOL_S = {torch.bfloat16: 1e-2, torch.float32: 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host32(t):
    return t.detach().float().cpu().numpy()


def lanes_view(t, last_dims):
    """[B,H,...] -> [B*H, ...] as fp32 numpy."""
    a = host32(t)
    return a.reshape((-1,) + a.shape[2:]) if last_dims else a.reshape(-1, a.shape[-1])


def oracle_prefill(q, k, v, la, beta, S0=None, lanes=None, rows=None):
    """fp64 oracle on lanes (flat b*H+h indices, or all). Returns (o, S_T) as float64 arrays."""
    qq, kk, vv, ll = (lanes_view(x, True) for x in (q, k, v, la))
    bb = host32(beta).reshape(-1, beta.shape[-1])
    ss = None if S0 is None else host32(S0).reshape(-1, S0.shape[-2], S0.shape[-1])
    if lanes is not None:
        qq, kk, vv, ll, bb = (x[lanes] for x in (qq, kk, vv, ll, bb))
        ss = None if ss is None else ss[lanes]
    return native.kda_fwd(qq, kk, vv, ll, bb, ss, rows=rows)


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def rel_l2_per_lane(S, S_ref):
    S = np.asarray(S, np.float64).reshape(S_ref.shape[0], -1)
    R = np.asarray(S_ref, np.float64).reshape(S_ref.shape[0], -1)
    num = np.linalg.norm(S - R, axis=1)
    den = np.linalg.norm(R, axis=1)
    return float(np.max(np.where(den > 0, num / np.maximum(den, 1e-300), num)))


def assert_close(tag, dtype, o_gpu, o_ref, S_gpu=None, S_ref=None):
    eo = max_abs(o_gpu, o_ref)
    msg = "%s: max|o-o_ref| = %.3e (tol %.0e)" % (tag, eo, TOL_O[dtype])
    ok = eo <= TOL_O[dtype]
    if S_gpu is not None:
        es = rel_l2_per_lane(S_gpu, S_ref)
        msg += ", relL2(S) = %.3e (tol %.0e)" % (es, TOL_S[dtype])
        ok = ok and es <= TOL_S[dtype]
    say(msg)
    assert ok, msg
