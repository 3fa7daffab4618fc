"""The elementwise steps on either side of the KDA core, in numpy fp64. Test infrastructure only.

Section 2.2 of the Kimi K3 reading notes (liuzhao09.github.io/papers/kimi-k3.html):
  - decay lower-bound equation: the per-head log decay is g = g_min * Sigmoid(e^{A_h} z) with the
    head-wise log scale A_h and the decay pre-activation z, alpha = exp(g), g_min = -5;
  - output gate equation: y = W_o [Sigmoid(W_g x) * RMSNorm(o~)], the RMSNorm taken per head.
Only the elementwise parts are here (W_g x arrives as `gate`, W_o is not applied). RMSNorm of a
head's output row o (dv values) is o / sqrt(mean(o^2) + eps) times a weight vector w.
"""
import numpy as np


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def log_decay(z, A_log, g_min=-5.0):
    """g = g_min * sigmoid(exp(A_log) * z); A_log broadcasts against z (one value per head)."""
    return float(g_min) * sigmoid(np.exp(np.asarray(A_log, dtype=np.float64)) * np.asarray(z, dtype=np.float64))


def gated_rmsnorm(o, gate, weight=None, eps=1e-6):
    """y = sigmoid(gate) * weight * o / sqrt(mean(o^2 over the last axis) + eps)."""
    o = np.asarray(o, dtype=np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    w = 1.0 if weight is None else np.asarray(weight, dtype=np.float64)
    return sigmoid(gate) * w * o / np.sqrt(ms + eps)
