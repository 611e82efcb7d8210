"""Seeded synthetic inputs for the KDA forward pass (tests and benchmark).

This module only draws random tensors; it holds none of the attention
arithmetic.  It serves both the GPU path and the oracle: the oracle always
receives host copies of exactly the tensors the GPU path consumed.

Workloads (shapes and distributions; the pages measure whole-model runs at
up to 1M tokens of context, these synthetic inputs stand in for them):
  * ``tiny_f32``        1 x 64 tokens, H=2, d=16, fp32 q/k/v, zero state
  * ``batch4_t4096``    4 x 4096 tokens, H=16, d=128, bf16, zero state
  * ``long_t1m``        1 x 1,048,576 tokens, H=32, d=128, bf16, zero state
  * ``decode_n256``     256 sequences x H=32, d=128, fp32 state ~ N(0, 0.02),
                        64 decode steps of one bf16 token each
  * ``varlen_n64``      64 sequences, lengths log-uniform in [128, 32768],
                        H=32, d=128, bf16, initial states ~ N(0, 0.02)
Distributions: q, k ~ N(0,1) then L2-normalised per (token, head) in fp32
and rounded to the storage dtype; v ~ N(0,1); beta = sigmoid(N(0,1));
log_alpha = -U(0.001, 0.1) ("uniform" gates) or -0.05*softplus(N(0,1))
("softplus" gates), drawn per (token, head, key channel).

Every tensor has its own stream, seeded from (seed, tensor id, slab), and
large tensors are drawn in fixed slabs of tokens, so a tensor's values do
not depend on how much else is generated.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

# tensor ids of the seeded streams
Q, K, V, LOG_ALPHA, BETA, STATE, LENGTHS, DO, DHT = range(9)   # DO, DHT: adjoints of o and hT
SLAB = 1 << 16   # tokens per generation slab


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" | "decode"
    N: int
    T: int               # tokens per sequence (prefill, fixed length) or 0 (varlen)
    H: int
    dk: int
    dv: int
    dtype: str           # "bf16" | "f32"
    gate: str            # "uniform" | "softplus"
    state_std: float     # 0 => zero initial state
    steps: int = 0       # decode steps
    varlen: tuple = field(default=())  # (lo, hi) of log-uniform lengths


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "prefill", 1, 64, 2, 16, 16, "f32", "uniform", 0.0),
    "batch4_t4096": Workload("batch4_t4096", "prefill", 4, 4096, 16, 128, 128, "bf16",
                             "uniform", 0.0),
    "long_t1m": Workload("long_t1m", "prefill", 1, 1 << 20, 32, 128, 128, "bf16",
                         "softplus", 0.0),
    "decode_n256": Workload("decode_n256", "decode", 256, 0, 32, 128, 128, "bf16",
                            "uniform", 0.02, steps=64),
    "varlen_n64": Workload("varlen_n64", "prefill", 64, 0, 32, 128, 128, "bf16",
                           "softplus", 0.02, varlen=(128, 32768)),
}


def torch_dtype(name: str):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _gen(seed: int, tensor: int, slab: int, device) -> torch.Generator:
    ss = np.random.SeedSequence([int(seed), int(tensor), int(slab)])
    g = torch.Generator(device=device)
    g.manual_seed(int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1)))
    return g


def _slabbed(shape, seed, tensor, device, draw):
    """Fill a [T, ...] fp32 tensor slab by slab with draw(gen, shape)."""
    out = torch.empty(shape, dtype=torch.float32, device=device)
    T = shape[0]
    for si, a in enumerate(range(0, T, SLAB)):
        b = min(T, a + SLAB)
        out[a:b] = draw(_gen(seed, tensor, si, device), (b - a,) + tuple(shape[1:]))
    return out


def _normal(g, shape, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def unit_rows(shape, seed, tensor, device, dtype):
    """N(0,1) rows L2-normalised along the last axis (fp32), then stored."""
    def draw(g, s):
        x = _normal(g, s, device)
        return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    return _slabbed(shape, seed, tensor, device, draw).to(dtype)


def normal(shape, seed, tensor, device, dtype, std=1.0):
    x = _slabbed(shape, seed, tensor, device, lambda g, s: _normal(g, s, device))
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def gates(shape, seed, device, kind):
    if kind == "uniform":
        def draw(g, s):
            u = torch.rand(s, generator=g, device=device, dtype=torch.float32)
            return -(0.001 + 0.099 * u)
    elif kind == "softplus":
        def draw(g, s):
            return -0.05 * torch.nn.functional.softplus(_normal(g, s, device))
    else:
        raise ValueError(kind)
    return _slabbed(shape, seed, LOG_ALPHA, device, draw)


def write_strength(shape, seed, device):
    return _slabbed(shape, seed, BETA, device, lambda g, s: torch.sigmoid(_normal(g, s, device)))


def varlen_lengths(n: int, lo: int, hi: int, seed: int):
    """Lengths log-uniform in [lo, hi]: round(exp(U(ln lo, ln hi))), clipped."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, LENGTHS])))
    L = np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), n))).astype(np.int64)
    return np.clip(L, lo, hi)


def prefill_inputs(lengths, H, dk, dv, dtype="bf16", gate="uniform", state_std=0.0,
                   seed=0, device="cpu"):
    """Packed prefill inputs for sequences of the given lengths.

    Returns a dict with q, k [T,H,dk], v [T,H,dv] (dtype), log_alpha
    [T,H,dk] fp32, beta [T,H] fp32, h0 [N,H,dk,dv] fp32 or None,
    cu_seqlens int32 [N+1] and the host list of lengths."""
    lengths = [int(x) for x in lengths]
    T = int(sum(lengths))
    dt = torch_dtype(dtype)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32,
                      device=device)
    d = dict(
        q=unit_rows((T, H, dk), seed, Q, device, dt),
        k=unit_rows((T, H, dk), seed, K, device, dt),
        v=normal((T, H, dv), seed, V, device, dt),
        log_alpha=gates((T, H, dk), seed, device, gate),
        beta=write_strength((T, H), seed, device),
        h0=None,
        cu_seqlens=cu,
        lengths=lengths,
    )
    if state_std > 0:
        d["h0"] = normal((len(lengths), H, dk, dv), seed, STATE, device, torch.float32,
                         std=state_std)
    return d


def workload_prefill_inputs(w: Workload, seed=0, device="cpu"):
    if w.varlen:
        lengths = varlen_lengths(w.N, w.varlen[0], w.varlen[1], seed)
    else:
        lengths = [w.T] * w.N
    return prefill_inputs(lengths, w.H, w.dk, w.dv, w.dtype, w.gate, w.state_std, seed, device)


def decode_state(N, H, dk, dv, std=0.02, seed=0, device="cpu"):
    return normal((N, H, dk, dv), seed, STATE, device, torch.float32, std=std)


def decode_token_inputs(N, H, dk, dv, dtype="bf16", gate="uniform", seed=0, step=0,
                        device="cpu"):
    """One decode token per sequence for the given step (fresh draws per step)."""
    s = int(np.random.SeedSequence([seed, 1000 + step]).generate_state(1)[0])
    dt = torch_dtype(dtype)
    return dict(
        q=unit_rows((N, H, dk), s, Q, device, dt),
        k=unit_rows((N, H, dk), s, K, device, dt),
        v=normal((N, H, dv), s, V, device, dt),
        log_alpha=gates((N, H, dk), s, device, gate),
        beta=write_strength((N, H), s, device),
    )
