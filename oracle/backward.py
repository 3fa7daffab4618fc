"""Gradient of the KDA recurrence, by reverse-mode differentiation of the token loop, in numpy
fp64. Test infrastructure only.

The forward is the state equation of section 2.2 of the Kimi K3 reading notes
(liuzhao09.github.io/papers/kimi-k3.html); the pages mention that training uses chunkwise KDA but
print no backward, so this is the plain derivative of that recurrence. Per token, written as the
steps the forward takes:
    Sbar_t = Diag(alpha_t) S_{t-1}            alpha_t = exp(log_alpha_t)
    r_t    = Sbar_t^T k_t                     prediction from the decayed state
    d_t    = beta_t (v_t - r_t)               the correction
    S_t    = Sbar_t + k_t d_t^T
    o_t    = S_t^T q_t
For a loss L with dL/do_t = do_t and dL/dS_T = dS_T, walking t backwards with G = dL/dS_t:
    G      += q_t do_t^T                      (o_t reads S_t)
    dq_t    = S_t do_t
    dd      = G^T k_t,   dk_t = G d_t
    dbeta_t = dd . (v_t - r_t),   dv_t = beta_t dd,   dr = -beta_t dd
    dSbar   = G + k_t dr^T,       dk_t += Sbar_t dr
    dlog_alpha_t[i] = sum_j dSbar[i, j] Sbar_t[i, j]      (d alpha_i / d log_alpha_i = alpha_i)
    G       = Diag(alpha_t) dSbar                        (= dL/dS_{t-1})
and dS_0 = G at the end. One lane at a time; every forward state is kept (small inputs only).
"""
import numpy as np


def kda_bwd_lane(q, k, v, log_alpha, beta, S0, do, dST):
    """One lane. q,k,log_alpha [T,dk]; v,do [T,dv]; beta [T]; S0, dST [dk,dv] (None = zeros).
    Returns dq, dk, dv, dlog_alpha, dbeta, dS0 (float64)."""
    q, k, v, la, beta, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, log_alpha, beta, do))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    alpha = np.exp(la)
    Sbar = np.empty((T, dk, dv))
    Ss = np.empty((T, dk, dv))
    r = np.empty((T, dv))
    d = np.empty((T, dv))
    for t in range(T):                       # forward, keeping what the backward reads
        Sbar[t] = alpha[t][:, None] * S
        r[t] = Sbar[t].T @ k[t]
        d[t] = beta[t] * (v[t] - r[t])
        S = Sbar[t] + np.outer(k[t], d[t])
        Ss[t] = S
    G = np.zeros((dk, dv)) if dST is None else np.array(dST, dtype=np.float64)
    dq = np.zeros_like(q)
    dk_ = np.zeros_like(k)
    dv_ = np.zeros_like(v)
    dla = np.zeros_like(la)
    dbeta = np.zeros_like(beta)
    for t in range(T - 1, -1, -1):
        G = G + np.outer(q[t], do[t])
        dq[t] = Ss[t] @ do[t]
        dd = G.T @ k[t]
        dk_[t] = G @ d[t]
        dbeta[t] = dd @ (v[t] - r[t])
        dv_[t] = beta[t] * dd
        dr = -beta[t] * dd
        dSbar = G + np.outer(k[t], dr)
        dk_[t] += Sbar[t] @ dr
        dla[t] = np.sum(dSbar * Sbar[t], axis=1)
        G = alpha[t][:, None] * dSbar
    return dq, dk_, dv_, dla, dbeta, G


def kda_bwd(q, k, v, log_alpha, beta, S0, do, dST):
    """Lanes stacked on axis 0 (shapes of kda_bwd_lane with a leading L); S0 / dST may be None."""
    L = np.shape(q)[0]
    outs = [kda_bwd_lane(q[l], k[l], v[l], log_alpha[l], beta[l], None if S0 is None else S0[l], do[l],
                         None if dST is None else dST[l]) for l in range(L)]
    return tuple(np.stack([o[i] for o in outs]) for i in range(6))
