"""Seeded synthetic inputs for the KDA workloads.

This module holds the input recipes only -- random draws, the L2
normalisation of q and k that the model applies before the operator, and
rounding to the storage dtype.  It contains none of the KDA arithmetic and is
shared by the tests (GPU path and oracle alike), the smoke check and the
benchmark.

Recipes (one numpy Generator per problem, seeded; draw order: sequence
lengths, q, k, v, g, beta, initial state; all draws in float32):
  q, k  ~ N(0, 1), then L2-normalised over the key channels of each
          (token, head) in float32, then rounded to the storage dtype
  v     ~ N(0, 1), rounded to the storage dtype
  g     = -5 * sigmoid(z), z ~ N(mu_g, 1) per (token, head, channel), fp32;
          mu_g = 0, or 2 for the near-bound workload.  g lies in [-5, 0]
          (the log-decay lower bound of "Two Paths: Kimi K3 vs DeepSeek V4
          Architecture Divergence", section "Hardware Adaptation").
  beta  = sigmoid(N(0, 1)) per (token, head), fp32
  S0    ~ N(0, 0.02^2) (std 0.02), fp32, or absent (zero state)
bf16 rounding is round-to-nearest-even on the float32 bit pattern.

`make_device` draws the same recipe directly on the GPU with torch's seeded
generator (a different random stream, the same distributions, shapes and
sequence lengths): the benchmark uses it for its largest workloads, whose
host-side draws take about a minute each.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# The five workloads (shapes of Kimi K3's KDA layers: 96 heads, head dim 128).
WORKLOADS = {
    "tiny": dict(kind="prefill", B=1, H=2, T=64, K=16, V=16, C=16,
                 dtype="fp32", g_mu=0.0, s0=False),
    "decode": dict(kind="decode", B=64, H=96, K=128, V=128, C=64,
                   dtype="bf16", g_mu=0.0, s0=True),
    "prefill": dict(kind="prefill", B=1, H=96, T=8192, K=128, V=128, C=64,
                    dtype="bf16", g_mu=0.0, s0=False),
    "long": dict(kind="prefill", B=1, H=32, T=131072, K=128, V=128, C=64,
                 dtype="bf16", g_mu=2.0, s0=True),
    "varlen": dict(kind="varlen", N=8, H=96, K=128, V=128, C=64,
                   dtype="bf16", g_mu=0.0, s0=True, len_lo=1024,
                   len_hi=16384),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 values exactly representable in bf16 (RNE)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of float32 values that are already bf16-exact."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


@dataclasses.dataclass
class Problem:
    """One synthetic KDA call.  Arrays are float32 holding the exact values
    of the storage dtype (bf16 values are bf16-rounded float32).

    prefill: q,k,g [B,T,H,K]; v [B,T,H,V]; beta [B,T,H]; S0 [B,H,K,V]
    varlen : q,k,g [total_T,H,K]; v [total_T,H,V]; beta [total_T,H];
             cu_seqlens [N+1] int32; S0 [N,H,K,V]
    decode : q,k,g [B,H,K]; v [B,H,V]; beta [B,H]; S0 [B,H,K,V] (required)
    """
    name: str
    kind: str
    dtype: str           # storage dtype of q, k, v and o: "bf16" or "fp32"
    H: int
    K: int
    V: int
    C: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    initial_state: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray] = None
    B: int = 0
    T: int = 0
    N: int = 0

    @property
    def tokens(self) -> int:
        if self.kind == "varlen":
            return int(self.cu_seqlens[-1])
        if self.kind == "decode":
            return self.B
        return self.B * self.T

    @property
    def seq_lengths(self):
        if self.kind == "varlen":
            return np.diff(self.cu_seqlens).astype(np.int64)
        if self.kind == "decode":
            return np.ones(self.B, np.int64)
        return np.full(self.B, self.T, np.int64)


def _sigmoid(z):
    return (np.float32(1) / (np.float32(1) + np.exp(-z))).astype(np.float32)


def _unit(x):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def make(name: str, seed: int = 0, **overrides) -> Problem:
    """Build workload ``name`` (a key of WORKLOADS) with optional size
    overrides (B, T, H, K, V, C, N, dtype, g_mu, s0, lengths, g_const,
    beta_const)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    rng = np.random.default_rng(seed)
    kind = cfg["kind"]
    H, K, V = cfg["H"], cfg["K"], cfg["V"]
    cu = None
    if kind == "varlen":
        if "lengths" in cfg:
            lengths = np.asarray(cfg["lengths"], np.int64)
        else:
            lengths = rng.integers(cfg["len_lo"], cfg["len_hi"] + 1,
                                   size=cfg["N"])
        cu = np.zeros(len(lengths) + 1, np.int32)
        cu[1:] = np.cumsum(lengths)
        lead = (int(cu[-1]),)
        nseq = len(lengths)
    elif kind == "decode":
        lead = (cfg["B"],)
        nseq = cfg["B"]
    else:
        lead = (cfg["B"], cfg["T"])
        nseq = cfg["B"]

    def normal(shape):
        return rng.standard_normal(shape, dtype=np.float32)

    store = bf16_round if cfg["dtype"] == "bf16" else (lambda x: x)
    q = store(_unit(normal(lead + (H, K))))
    k = store(_unit(normal(lead + (H, K))))
    v = store(normal(lead + (H, V)))
    g = (np.float32(-5) * _sigmoid(normal(lead + (H, K)) +
                                   np.float32(cfg["g_mu"]))).astype(np.float32)
    beta = _sigmoid(normal(lead + (H,)))
    s0 = None
    if cfg["s0"]:
        s0 = (np.float32(0.02) * normal((nseq, H, K, V))).astype(np.float32)
    if "g_const" in cfg:
        g = np.full_like(g, np.float32(cfg["g_const"]))
    if "beta_const" in cfg:
        beta = np.full_like(beta, np.float32(cfg["beta_const"]))
    return Problem(name=name, kind=kind, dtype=cfg["dtype"], H=H, K=K, V=V,
                   C=cfg["C"], q=q, k=k, v=v, g=g, beta=beta,
                   initial_state=s0, cu_seqlens=cu,
                   B=cfg.get("B", 0), T=cfg.get("T", 0),
                   N=nseq if kind == "varlen" else 0)


def varlen_lengths(name: str, seed: int = 0, **overrides) -> np.ndarray:
    """The sequence lengths `make` draws for a varlen workload (its first
    draw from the seeded generator)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    if "lengths" in cfg:
        return np.asarray(cfg["lengths"], np.int64)
    rng = np.random.default_rng(seed)
    return rng.integers(cfg["len_lo"], cfg["len_hi"] + 1, size=cfg["N"])


def make_device(name: str, seed: int, device, **overrides) -> dict:
    """Workload ``name`` drawn on ``device`` with torch (recipe as `make`).
    Returns a dict of device tensors q, k, v, g, beta, initial_state (or
    None) and cu_seqlens (int32, also for fixed-length workloads: B
    sequences of T tokens), plus the sizes."""
    import torch
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    kind = cfg["kind"]
    if kind == "decode":
        raise ValueError("make_device covers the prefill workloads")
    H, K, V = cfg["H"], cfg["K"], cfg["V"]
    if kind == "varlen":
        lengths = varlen_lengths(name, seed, **overrides)
    else:
        lengths = np.full(cfg["B"], cfg["T"], np.int64)
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    total = int(cu[-1])
    gen = torch.Generator(device=device).manual_seed(int(seed))
    dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32

    def normal(*shape):
        return torch.randn(shape, generator=gen, device=device,
                           dtype=torch.float32)

    def unit(x):
        return x / torch.sqrt(torch.sum(x * x, dim=-1, keepdim=True))

    q = unit(normal(total, H, K)).to(dt)
    k = unit(normal(total, H, K)).to(dt)
    v = normal(total, H, V).to(dt)
    g = -5.0 * torch.sigmoid(normal(total, H, K) + float(cfg["g_mu"]))
    beta = torch.sigmoid(normal(total, H))
    s0 = 0.02 * normal(len(lengths), H, K, V) if cfg["s0"] else None
    return dict(name=name, q=q, k=k, v=v, g=g, beta=beta, initial_state=s0,
                cu_seqlens=torch.from_numpy(cu).to(device), lengths=lengths,
                H=H, K=K, V=V, C=cfg["C"], dtype=cfg["dtype"], total=total)
