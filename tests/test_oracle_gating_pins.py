"""Pins of the oracle's fused prologue / epilogue functions (CPU only): closed forms of the decay
lower-bound equation and of the per-head RMSNorm with sigmoid output gate (section 2.2 of the Kimi
K3 reading notes, liuzhao09.github.io/papers/kimi-k3.html), and planted slips that must fail them."""
import math

import numpy as np

from oracle import gating


def _decay_pins(fn):
    """fn(z, A_log, g_min) -> g. True when every closed form holds."""
    ok = True
    # z = 0: sigmoid(0) = 1/2, whatever A
    ok &= abs(fn(0.0, 0.7, -5.0) - (-2.5)) < 1e-15
    # exp(A) z = ln 3 -> sigmoid = 3/4: A = ln 2, z = ln(3) / 2 (the head scale enters through exp)
    ok &= abs(fn(math.log(3.0) / 2, math.log(2.0), -5.0) - (-3.75)) < 1e-14
    # the bound: g -> g_min for z -> +inf, g -> 0 for z -> -inf, strictly inside (g_min, 0)
    ok &= abs(fn(60.0, 0.0, -5.0) - (-5.0)) < 1e-12 and abs(fn(-60.0, 0.0, -5.0)) < 1e-12
    zs = np.linspace(-8, 8, 101)
    g = np.array([fn(z, 0.3, -5.0) for z in zs])
    ok &= bool(np.all(g < 0) and np.all(g > -5.0) and np.all(np.diff(g) < 0))   # decreasing in z
    # g_min scales the result
    ok &= abs(fn(0.4, -0.2, -2.0) * 2.5 - fn(0.4, -0.2, -5.0)) < 1e-14
    return bool(ok)


def _norm_pins(fn):
    """fn(o, gate, weight, eps) -> y. True when every closed form holds."""
    ok = True
    # o = (3, 4): mean(o^2) = 12.5; gate 0 -> sigmoid 1/2; y = (3, 4) / (2 sqrt(12.5))
    y = fn(np.array([3.0, 4.0]), np.array([0.0, 0.0]), None, 0.0)
    ok &= bool(np.allclose(y, [0.42426406871192851, 0.56568542494923802], rtol=0, atol=1e-15))
    # weight multiplies per column; a large gate passes the normalised row
    y = fn(np.array([3.0, 4.0]), np.array([50.0, 50.0]), np.array([2.0, -1.0]), 0.0)
    ok &= bool(np.allclose(y, [2 * 3 / math.sqrt(12.5), -4 / math.sqrt(12.5)], rtol=0, atol=1e-12))
    # scale invariance with eps = 0 and a unit root mean square after normalisation
    rng = np.random.default_rng(3)
    o = rng.standard_normal((5, 16))
    gate = np.full((5, 16), 60.0)
    y1, y2 = fn(o, gate, None, 0.0), fn(7.5 * o, gate, None, 0.0)
    ok &= bool(np.allclose(y1, y2, rtol=1e-13, atol=0)) and bool(np.allclose(np.mean(y1 * y1, axis=-1), 1.0, rtol=1e-12))
    # eps enters under the square root: o = 0 stays 0, and a tiny row is damped
    ok &= bool(np.all(fn(np.zeros(4), np.zeros(4), None, 1e-6) == 0))
    y = fn(np.array([1e-3, 1e-3]), np.array([60.0, 60.0]), None, 1e-6)
    ok &= bool(np.allclose(y, 1e-3 / math.sqrt(1e-6 + 1e-6), rtol=1e-12))
    return bool(ok)


def test_decay_prologue_closed_forms():
    assert _decay_pins(lambda z, A, gm: float(gating.log_decay(z, A, gm)))


def test_gated_rmsnorm_closed_forms():
    assert _norm_pins(lambda o, g, w, e: gating.gated_rmsnorm(o, g, w, e))


def test_planted_slips_fail_the_pins():
    sig = gating.sigmoid
    decay_slips = {
        "no exp on A": lambda z, A, gm: gm * float(sig(A * z)),
        "sign of z": lambda z, A, gm: gm * float(sig(-math.exp(A) * z)),
        "g_min dropped": lambda z, A, gm: -float(sig(math.exp(A) * z)),
        "tanh for sigmoid": lambda z, A, gm: gm * math.tanh(math.exp(A) * z),
    }
    for name, fn in decay_slips.items():
        assert not _decay_pins(fn), name

    def rms(o, eps, use_sum=False, sqrt=True):
        m = np.sum(o * o, axis=-1, keepdims=True) if use_sum else np.mean(o * o, axis=-1, keepdims=True)
        return np.sqrt(m + eps) if sqrt else m + eps

    w1 = lambda w: 1.0 if w is None else w
    norm_slips = {
        "sum for mean": lambda o, g, w, e: sig(g) * w1(w) * o / rms(o, e, use_sum=True),
        "no square root": lambda o, g, w, e: sig(g) * w1(w) * o / rms(o, e, sqrt=False),
        "no gate sigmoid": lambda o, g, w, e: g * w1(w) * o / rms(o, e),
        "eps outside the root": lambda o, g, w, e: sig(g) * w1(w) * o / (rms(o, 0.0) + e),
        "weight dropped": lambda o, g, w, e: sig(g) * o / rms(o, e),
    }
    for name, fn in norm_slips.items():
        assert not _norm_pins(fn), name
