"""Chunkwise KDA in numpy fp64. Test infrastructure only.

Follows the chunk equations of section 2.2 of the Kimi K3 reading notes
(liuzhao09.github.io/papers/kimi-k3.html), in the pages' notation, for one chunk with entry
state S and rows r = 1..C:

  cumulative decay      gamma^{i->j} = prod_{r=i..j} alpha^r ; row r of Gamma is gamma^{1->r}
  UT transform          builds U (C x d_v), W (C x d_k); pseudo-value  V~ = U - W S
  causal matrix         A = Tril[(Q*Gamma)(K/Gamma)^T]   (lower triangle including the diagonal)
  output                O = (Gamma*Q) S + A V~

The pages name U and W but do not print them, nor the chunk-end state. Unrolling the
recurrence inside a chunk (S_r = Gamma_r S + sum_{j<=r} (Gamma_r/Gamma_j) k_j u_j^T) gives:

  A_kk = Diag(beta) StrictTril[(K*Gamma)(K/Gamma)^T]
  U    = (I + A_kk)^{-1} Diag(beta) V
  W    = (I + A_kk)^{-1} Diag(beta) (K*Gamma)
  S'   = Diag(gamma^{1->C}) S + (K * gamma^{1->C}/Gamma)^T V~

and the affine pair of section 2.5 for a chunk, S_out = S~ + M S_in, with
  M  = Diag(gamma^{1->C}) - (K * gamma^{1->C}/Gamma)^T W,     S~ = (K * gamma^{1->C}/Gamma)^T U.

A ragged last chunk simply has fewer rows. Triangular solves use scipy (a library primitive).
"""
import numpy as np
from scipy.linalg import solve_triangular


def _chunk_pieces(k, v, la, beta):
    G = np.cumsum(la, axis=0)                  # log gamma^{1->r}, row r
    Gam = np.exp(G)
    Kg = k * Gam                               # K * Gamma
    Kinv = k / Gam                             # K / Gamma
    Kbar = k * np.exp(G[-1] - G)               # K * gamma^{1->C} / Gamma
    n = k.shape[0]
    A_kk = beta[:, None] * np.tril(Kg @ Kinv.T, -1)
    IA = np.eye(n) + A_kk
    U = solve_triangular(IA, beta[:, None] * v, lower=True, unit_diagonal=True)
    W = solve_triangular(IA, beta[:, None] * Kg, lower=True, unit_diagonal=True)
    return G, Gam, Kinv, Kbar, U, W


def kda_chunked(q, k, v, log_alpha, beta, S0=None, C=64):
    """Chunk form over lanes. Shapes as ``recurrence.kda_fwd``. Returns (o, S_T) float64."""
    q, k, v, la, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, log_alpha, beta))
    L, T, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((L, T, dv))
    ST = np.zeros((L, dk, dv))
    for l in range(L):
        S = np.zeros((dk, dv)) if S0 is None else np.array(S0[l], dtype=np.float64)
        for s in range(0, T, C):
            e = min(T, s + C)
            G, Gam, Kinv, Kbar, U, W = _chunk_pieces(k[l, s:e], v[l, s:e], la[l, s:e], beta[l, s:e])
            Qg = q[l, s:e] * Gam
            Vt = U - W @ S                                   # pseudo-value
            A = np.tril(Qg @ Kinv.T)                         # causal matrix incl. diagonal
            o[l, s:e] = Qg @ S + A @ Vt
            S = np.exp(G[-1])[:, None] * S + Kbar.T @ Vt
        ST[l] = S
    return o, ST


def segment_affine_pair(k, v, log_alpha, beta, C=64):
    """Affine pair (M, S~) of one lane's token range: S_out = S~ + M S_in (section 2.5).
    Built chunk by chunk: M <- M_c M, S~ <- M_c S~ + S~_c. Shapes: k, log_alpha [T,dk];
    v [T,dv]; beta [T]. Returns (M [dk,dk], S~ [dk,dv])."""
    k, v, la, beta = (np.asarray(a, dtype=np.float64) for a in (k, v, log_alpha, beta))
    T, dk = k.shape
    M = np.eye(dk)
    St = np.zeros((dk, v.shape[1]))
    for s in range(0, T, C):
        e = min(T, s + C)
        G, _, _, Kbar, U, W = _chunk_pieces(k[s:e], v[s:e], la[s:e], beta[s:e])
        Mc = np.diag(np.exp(G[-1])) - Kbar.T @ W
        M = Mc @ M
        St = Mc @ St + Kbar.T @ U
    return M, St


def compose_entry_states(pairs, S0):
    """Exact entry state of every segment from the segments' affine pairs, in order:
    entry_0 = S0, entry_{s+1} = S~_s + M_s entry_s. Returns the list of entries and the exit."""
    entries = []
    S = np.array(S0, dtype=np.float64)
    for M, St in pairs:
        entries.append(S)
        S = St + M @ S
    return entries, S
