"""KDA recurrence in exact rational arithmetic, for tiny inputs. Test infrastructure only.

The state equation of section 2.2 of the Kimi K3 reading notes
(liuzhao09.github.io/papers/kimi-k3.html) is evaluated literally as matrices of Fractions:
S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t.
Here alpha is given directly (rational), not through exp, so nothing is rounded.
"""
from fractions import Fraction


def _mat(rows, cols, f=lambda i, j: Fraction(0)):
    return [[f(i, j) for j in range(cols)] for i in range(rows)]


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][l] * B[l][j] for l in range(m)), Fraction(0)) for j in range(p)] for i in range(n)]


def kda_fwd(q, k, v, alpha, beta, S0=None):
    """q,k,alpha: T lists of dk Fractions; v: T lists of dv Fractions; beta: T Fractions.
    Returns (o as T lists of dv Fractions, S_T as dk x dv Fractions)."""
    T = len(k)
    dk = len(k[0])
    dv = len(v[0])
    S = _mat(dk, dv) if S0 is None else [list(map(Fraction, row)) for row in S0]
    outs = []
    for t in range(T):
        erase = _mat(dk, dk, lambda i, j: (Fraction(1) if i == j else Fraction(0)) - beta[t] * k[t][i] * k[t][j])
        decay = _mat(dk, dk, lambda i, j: alpha[t][i] if i == j else Fraction(0))
        write = _mat(dk, dv, lambda i, j: beta[t] * k[t][i] * v[t][j])
        S = _matmul(_matmul(erase, decay), S)
        S = [[S[i][j] + write[i][j] for j in range(dv)] for i in range(dk)]
        outs.append([sum((S[c][j] * q[t][c] for c in range(dk)), Fraction(0)) for j in range(dv)])
    return outs, S
