"""KDA recurrence in numpy fp64, vectorised over lanes. Test infrastructure only.

Follows the state equation of section 2.2 of the Kimi K3 reading notes
(liuzhao09.github.io/papers/kimi-k3.html): per head a d_k x d_v state,
S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T and o_t = S_t^T q_t,
alpha_t = exp(log_alpha_t) per key channel.
"""
import numpy as np


def kda_fwd(q, k, v, log_alpha, beta, S0=None):
    """Token loop. q,k,log_alpha [L,T,dk]; v [L,T,dv]; beta [L,T]; S0 [L,dk,dv] or None.
    Returns (o [L,T,dv], S_T [L,dk,dv]) in float64."""
    q, k, v, la, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, log_alpha, beta))
    L, T, dk = q.shape
    dv = v.shape[2]
    S = np.zeros((L, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((L, T, dv))
    for t in range(T):
        S = S * np.exp(la[:, t, :])[:, :, None]                      # Diag(alpha_t) S_{t-1}
        pred = np.einsum("lc,lcj->lj", k[:, t], S)                     # k_t^T (decayed S)
        S = S + beta[:, t, None, None] * k[:, t, :, None] * (v[:, t, None, :] - pred[:, None, :])
        o[:, t] = np.einsum("lc,lcj->lj", q[:, t], S)                 # S_t^T q_t
    return o, S


def transition(k_t, log_alpha_t, beta_t):
    """The per-token transition matrix Phi_t = (I - beta_t k_t k_t^T) Diag(alpha_t) of one lane,
    written as the product printed in the recurrence equation."""
    k_t = np.asarray(k_t, dtype=np.float64)
    dk = k_t.shape[0]
    return (np.eye(dk) - beta_t * np.outer(k_t, k_t)) @ np.diag(np.exp(np.asarray(log_alpha_t, np.float64)))


def kda_product_form(q, k, v, log_alpha, beta, S0):
    """One lane in product form: S_T = Phi_T...Phi_1 S_0 + sum_t Phi_T...Phi_{t+1} beta_t k_t v_t^T,
    built from explicit dense transition matrices. Returns (o [T,dv], S_T)."""
    q, k, v, la = (np.asarray(a, dtype=np.float64) for a in (q, k, v, log_alpha))
    T, dk = k.shape
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        S = transition(k[t], la[t], beta[t]) @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S
