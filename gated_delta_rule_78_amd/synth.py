"""Seeded synthetic inputs for the KDA workloads.

This module only draws random tensors with the workloads' shapes and value distributions; it
holds none of the method's arithmetic. Both the HIP path's tests and the oracle's tests take
their inputs from here (the oracle receives host copies of exactly these tensors).

Value recipe (per (b,h) lane, seeded with ``seed_base + b*H + h``):
  q, k      ~ N(0,1), then L2-normalised over the key dimension per token (in fp32), then cast
  v         ~ N(0,1)
  log_alpha ~ U[lo, hi] per key channel (default U[-0.5, -0.001])
  beta      = sigmoid(N(0,1)) per token
  S0        ~ N(0, std) in fp32 when a carried prefix state is wanted
"""
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

LOG_ALPHA_RANGE = (-0.5, -0.001)


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    H: int
    T: int
    d: int
    dtype: torch.dtype
    s0_std: Optional[float] = None


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    N: int
    H: int
    d: int
    steps: int
    s_std: float
    dtype: torch.dtype = torch.bfloat16


# The five synthetic workloads of the KDA hot path.
PREFILL_FP32_SMALL = PrefillWorkload("prefill fp32 B=1 H=1 T=256 d=64 C=64", 1, 1, 256, 64, torch.float32)
PREFILL_BF16_8K = PrefillWorkload("prefill bf16 B=1 H=32 T=8192 d=128 C=64", 1, 32, 8192, 128, torch.bfloat16)
PREFILL_BF16_PREFIX_64K = PrefillWorkload("prefill bf16 +S0 B=4 H=32 T=65536 d=128 C=64", 4, 32, 65536, 128,
                                          torch.bfloat16, s0_std=0.02)
DECODE_BF16_256x32 = DecodeWorkload("decode bf16 N=256 H=32 d=128 fp32 state, 1000 chained steps", 256, 32, 128,
                                    1000, 0.02)
PREFILL_BF16_1M = PrefillWorkload("prefill bf16 B=1 H=32 T=1048576 d=128 C=64 (sequence split)", 1, 32, 1 << 20,
                                  128, torch.bfloat16)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def lane_inputs(T: int, dk: int, dv: int, dtype, seed: int, device="cpu",
                log_alpha_range: Tuple[float, float] = LOG_ALPHA_RANGE):
    """One lane's (q, k, v, log_alpha, beta): [T,dk], [T,dk], [T,dv], [T,dk], [T]."""
    g = _gen(device, seed)
    lo, hi = log_alpha_range
    q = torch.randn(T, dk, generator=g, device=device, dtype=torch.float32)
    q = q / q.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    k = torch.randn(T, dk, generator=g, device=device, dtype=torch.float32)
    k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    v = torch.randn(T, dv, generator=g, device=device, dtype=torch.float32)
    la = torch.rand(T, dk, generator=g, device=device, dtype=torch.float32) * (lo - hi) + hi
    beta = torch.sigmoid(torch.randn(T, generator=g, device=device, dtype=torch.float32))
    return tuple(x.to(dtype) for x in (q, k, v, la, beta))


def prefill_inputs(B: int, H: int, T: int, dk: int, dv: int, dtype, device="cpu", seed_base: int = 1000,
                   s0_std: Optional[float] = None, log_alpha_range: Tuple[float, float] = LOG_ALPHA_RANGE):
    """Stacked inputs: q,k,log_alpha [B,H,T,dk]; v [B,H,T,dv]; beta [B,H,T]; S0 [B,H,dk,dv] fp32 or None."""
    q = torch.empty(B, H, T, dk, dtype=dtype, device=device)
    k = torch.empty_like(q)
    la = torch.empty_like(q)
    v = torch.empty(B, H, T, dv, dtype=dtype, device=device)
    beta = torch.empty(B, H, T, dtype=dtype, device=device)
    S0 = None
    if s0_std is not None:
        S0 = torch.empty(B, H, dk, dv, dtype=torch.float32, device=device)
    for b in range(B):
        for h in range(H):
            seed = seed_base + b * H + h
            lq, lk, lv, lla, lb = lane_inputs(T, dk, dv, dtype, seed, device, log_alpha_range)
            q[b, h], k[b, h], v[b, h], la[b, h], beta[b, h] = lq, lk, lv, lla, lb
            if S0 is not None:
                S0[b, h] = torch.randn(dk, dv, generator=_gen(device, seed + 7_000_000), device=device,
                                       dtype=torch.float32) * s0_std
    return q, k, v, la, beta, S0


def workload_inputs(w: PrefillWorkload, device="cpu", seed_base: int = 1000, T: Optional[int] = None,
                    log_alpha_range: Tuple[float, float] = LOG_ALPHA_RANGE):
    """Inputs of a named prefill workload (optionally with a shorter T)."""
    return prefill_inputs(w.B, w.H, w.T if T is None else T, w.d, w.d, w.dtype, device, seed_base,
                          w.s0_std, log_alpha_range)


# Packed batch standing in for a prefill batch of mixed request lengths: 8192 tokens per head in
# 12 sequences (lengths from a few tens to 2.5K, three of them multiples of 512, most ragged),
# 32 heads, d = 128, checkpoints every 512 tokens (the 512-token hash blocks of a prefix cache).
PACKED_BF16_8K_LENS = (2500, 1536, 1024, 900, 700, 512, 413, 300, 150, 90, 40, 27)
PACKED_BF16_8K = PrefillWorkload("prefill bf16 packed 12 seqs (8192 tokens) H=32 d=128 C=64, checkpoints every 512",
                                 12, 32, 8192, 128, torch.bfloat16)


def packed_inputs(lens, H: int, dk: int, dv: int, dtype, device="cpu", seed_base: int = 5000,
                  s0_std: Optional[float] = None, log_alpha_range: Tuple[float, float] = LOG_ALPHA_RANGE):
    """A packed batch: sequence s (length lens[s]) is rows cu[s]..cu[s+1]-1 of every head.
    Returns q,k,log_alpha [H,T,dk]; v [H,T,dv]; beta [H,T]; cu_seqlens int32 [N+1];
    S0 [N,H,dk,dv] fp32 or None. Lane (s, h) is seeded with seed_base + s*H + h."""
    N = len(lens)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + int(n))
    T = cu[-1]
    q = torch.empty(H, T, dk, dtype=dtype, device=device)
    k = torch.empty_like(q)
    la = torch.empty_like(q)
    v = torch.empty(H, T, dv, dtype=dtype, device=device)
    beta = torch.empty(H, T, dtype=dtype, device=device)
    S0 = None if s0_std is None else torch.empty(N, H, dk, dv, dtype=torch.float32, device=device)
    for s in range(N):
        a, b = cu[s], cu[s + 1]
        for h in range(H):
            seed = seed_base + s * H + h
            lq, lk, lv, lla, lb = lane_inputs(b - a, dk, dv, dtype, seed, device, log_alpha_range)
            q[h, a:b], k[h, a:b], v[h, a:b], la[h, a:b], beta[h, a:b] = lq, lk, lv, lla, lb
            if S0 is not None:
                S0[s, h] = torch.randn(dk, dv, generator=_gen(device, seed + 7_000_000), device=device,
                                       dtype=torch.float32) * s0_std
    return q, k, v, la, beta, torch.tensor(cu, dtype=torch.int32, device=device), S0


def gating_inputs(lead, H: int, dk: int, dv: int, dtype, device="cpu", seed: int = 6000):
    """Inputs of the fused prologue / epilogue around the core, for rows shaped `lead` (e.g. (H, T)
    packed or (N, H) decode): z [*lead, dk] ~ N(-3, 1.5^2) (so that g = -5 sigmoid(e^A z) sits
    mostly in [-0.5, 0) with a tail toward -5), A_log [H] ~ U[-0.5, 0.5] fp32, gate [*lead, dv]
    ~ N(0, 1), norm_weight [dv] = 1 + 0.1 N(0, 1) fp32."""
    g = _gen(device, seed)
    z = (torch.randn(*lead, dk, generator=g, device=device) * 1.5 - 3.0).to(dtype)
    A_log = torch.rand(H, generator=g, device=device) - 0.5
    gate = torch.randn(*lead, dv, generator=g, device=device).to(dtype)
    w = 1.0 + 0.1 * torch.randn(dv, generator=g, device=device)
    return z, A_log, gate, w


def decode_state(N: int, H: int, dk: int, dv: int, std: float, device="cpu", seed: int = 3000):
    """Fixed-size fp32 state [N,H,dk,dv] ~ N(0, std)."""
    return torch.randn(N, H, dk, dv, generator=_gen(device, seed), device=device, dtype=torch.float32) * std


def decode_tokens(N: int, H: int, dk: int, dv: int, dtype, device="cpu", seed: int = 4000,
                  log_alpha_range: Tuple[float, float] = LOG_ALPHA_RANGE):
    """One decode step's token inputs: q,k,log_alpha [N,H,dk]; v [N,H,dv]; beta [N,H]."""
    g = _gen(device, seed)
    lo, hi = log_alpha_range
    q = torch.randn(N, H, dk, generator=g, device=device)
    q = q / q.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    k = torch.randn(N, H, dk, generator=g, device=device)
    k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    v = torch.randn(N, H, dv, generator=g, device=device)
    la = torch.rand(N, H, dk, generator=g, device=device) * (lo - hi) + hi
    beta = torch.sigmoid(torch.randn(N, H, generator=g, device=device))
    return tuple(x.to(dtype) for x in (q, k, v, la, beta))
