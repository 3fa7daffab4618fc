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


def check_lanes_streamed(tag, dtype, q, k, v, la, beta, S0, o, S_T, lanes, group=2):
    """Oracle parity on the given flat lanes (b*H + h) of one launch, `group` lanes at a time so that
    host memory stays bounded: every output row and the final state of each lane are compared.
    Returns (max|o - o_ref|, max rel-L2 of S) over the lanes; asserts the tolerances."""
    flat = lambda t: t.reshape((-1,) + tuple(t.shape[2:]))
    fq, fk, fv, fla, fb, fo, fS = (flat(x) for x in (q, k, v, la, beta, o, S_T))
    fS0 = None if S0 is None else flat(S0)
    worst_o, worst_s = 0.0, 0.0
    for i in range(0, len(lanes), group):
        sel = list(lanes[i:i + group])
        host = lambda t: None if t is None else t[sel].float().cpu().numpy()
        o_ref, S_ref = native.kda_fwd(host(fq), host(fk), host(fv), host(fla), host(fb), host(fS0))
        eo = max_abs(host(fo), o_ref)
        es = rel_l2_per_lane(host(fS), S_ref)
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
        say("%s: lanes %s max|o-o_ref| = %.3e relL2(S) = %.3e" % (tag, sel, eo, es))
        del o_ref, S_ref
        assert eo <= TOL_O[dtype] and es <= TOL_S[dtype], "%s: lanes %s out of tolerance" % (tag, sel)
    say("%s: %d lanes, every row: max|o-o_ref| = %.3e (tol %.0e), max relL2(S) = %.3e (tol %.0e)"
        % (tag, len(lanes), worst_o, TOL_O[dtype], worst_s, TOL_S[dtype]))
    return worst_o, worst_s
