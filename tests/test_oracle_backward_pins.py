"""Pins of the backward oracle (CPU only). The pages print no backward for chunkwise KDA (section
2.2 of the Kimi K3 reading notes, liuzhao09.github.io/papers/kimi-k3.html, says training uses it),
so the gradient is pinned to its definition: central finite differences of the fp64 forward, and
torch.autograd of a plain fp64 torch forward; plus a closed form, and planted slips that must fail
the finite-difference pin."""
import numpy as np
import torch

from oracle import backward, recurrence

RNG = np.random.default_rng(99)


def _inputs(T, dk, dv, L=1, rng=RNG, la_lo=-0.6):
    q = rng.standard_normal((L, T, dk))
    k = rng.standard_normal((L, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((L, T, dv))
    la = rng.uniform(la_lo, 0.0, (L, T, dk))
    beta = rng.uniform(0.1, 0.9, (L, T))
    S0 = 0.5 * rng.standard_normal((L, dk, dv))
    do = rng.standard_normal((L, T, dv))
    dST = rng.standard_normal((L, dk, dv))
    return q, k, v, la, beta, S0, do, dST


def _loss(q, k, v, la, beta, S0, do, dST):
    o, S = recurrence.kda_fwd(q, k, v, la, beta, S0)
    return float(np.sum(o * do) + np.sum(S * dST))


def _fd_pin(bwd, h=1e-6, tol=1e-7):
    """True when bwd matches central differences of the forward on a tiny case."""
    args = list(_inputs(6, 3, 2, rng=np.random.default_rng(5)))
    grads = bwd(*args)
    for gi, ai in zip(range(6), (0, 1, 2, 3, 4, 5)):   # q, k, v, log_alpha, beta, S0
        x = args[ai]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(*args)
            x[idx] = old - h
            lm = _loss(*args)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        if np.max(np.abs(num - grads[gi])) > tol * max(1.0, np.max(np.abs(num))):
            return False
    return True


def test_matches_central_differences():
    assert _fd_pin(backward.kda_bwd)


def test_matches_torch_autograd():
    q, k, v, la, beta, S0, do, dST = _inputs(40, 8, 6, L=2)
    tq, tk, tv, tla, tb, tS0 = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v, la, beta, S0))
    S = tS0
    outs = []
    for t in range(q.shape[1]):           # the recurrence, written plainly in torch
        A = torch.eye(8, dtype=torch.float64) - tb[:, t, None, None] * tk[:, t, :, None] * tk[:, t, None, :]
        S = A @ (torch.exp(tla[:, t])[:, :, None] * S) + tb[:, t, None, None] * tk[:, t, :, None] * tv[:, t, None, :]
        outs.append(torch.einsum("lc,lcj->lj", tq[:, t], S))
    loss = (torch.stack(outs, 1) * torch.tensor(do)).sum() + (S * torch.tensor(dST)).sum()
    loss.backward()
    ref = [x.grad.numpy() for x in (tq, tk, tv, tla, tb, tS0)]
    got = backward.kda_bwd(q, k, v, la, beta, S0, do, dST)
    for name, a, b in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"), got, ref):
        assert np.max(np.abs(a - b)) < 1e-10 * max(1.0, np.max(np.abs(b))), name


def test_no_decay_no_write_closed_form():
    """alpha = 1, beta = 0: S_t = S0 for all t, so dq_t = S0 do_t, dS0 = dS_T + sum_t q_t do_t^T,
    dv = dk = 0 and dlog_alpha_t[i] = sum_j G_t[i, j] S0[i, j] with G_t = dS_T + sum_{t' >= t} q_t' do_t'^T."""
    q, k, v, la, beta, S0, do, dST = _inputs(9, 4, 3)
    la[:] = 0.0
    beta[:] = 0.0
    dq, dk, dv, dla, dbeta, dS0 = backward.kda_bwd(q, k, v, la, beta, S0, do, dST)
    assert np.allclose(dq[0], do[0] @ S0[0].T, atol=1e-13)
    assert np.allclose(dS0[0], dST[0] + q[0].T @ do[0], atol=1e-12)
    assert np.all(dv == 0) and np.all(dk == 0)
    G = dST[0].copy()
    for t in range(8, -1, -1):
        G = G + np.outer(q[0, t], do[0, t])
        assert np.allclose(dla[0, t], np.sum(G * S0[0], axis=1), atol=1e-12)


def _slip(variant):
    def bwd(q, k, v, la, beta, S0, do, dST):
        outs = []
        for l in range(q.shape[0]):
            T, dk = k.shape[1:]
            S = S0[l].copy()
            alpha = np.exp(la[l])
            Sbar, Ss, r, d = [], [], [], []
            for t in range(T):
                Sb = alpha[t][:, None] * S
                rt = Sb.T @ k[l, t]
                dt = beta[l, t] * (v[l, t] - rt)
                S = Sb + np.outer(k[l, t], dt)
                Sbar.append(Sb); Ss.append(S); r.append(rt); d.append(dt)
            G = dST[l].copy()
            g = [np.zeros_like(x) for x in (q[l], k[l], v[l], la[l], beta[l])]
            for t in range(T - 1, -1, -1):
                if variant != "decay_before_read":
                    G = G + np.outer(q[l, t], do[l, t])
                g[0][t] = (Sbar[t] if variant == "dq_from_decayed" else Ss[t]) @ do[l, t]
                dd = G.T @ k[l, t]
                g[1][t] = G @ d[t]
                g[4][t] = dd @ (v[l, t] - r[t])
                g[2][t] = beta[l, t] * dd
                dr = -beta[l, t] * dd
                dSbar = G + np.outer(k[l, t], dr)
                if variant != "drop_prediction_path":
                    g[1][t] += Sbar[t] @ dr
                g[3][t] = np.sum((G if variant == "dlog_alpha_from_G" else dSbar) * Sbar[t], axis=1)
                G = alpha[t][:, None] * dSbar
                if variant == "decay_before_read":
                    G = G + alpha[t][:, None] * np.outer(q[l, t], do[l, t])
            outs.append(tuple(g) + (G,))
        return tuple(np.stack([o[i] for o in outs]) for i in range(6))
    return bwd


def test_real_slip_harness_passes_and_slips_fail():
    assert _fd_pin(_slip("none"))
    for variant in ("drop_prediction_path", "dq_from_decayed", "dlog_alpha_from_G", "decay_before_read"):
        assert not _fd_pin(_slip(variant)), variant
