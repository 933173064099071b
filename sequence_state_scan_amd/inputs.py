"""Seeded synthetic inputs for the GLA workloads (no method arithmetic lives here).

This module only draws random numbers and rounds them; the oracle and the HIP path both consume
its output and nothing else is shared between them.

Recipe (one ``numpy.random.default_rng(seed)`` stream, whole C-order tensors, in this order):

  q, k   ~ N(0,1) / sqrt(dk)    float32 draw, scaled in float32        shape [B,H,T,dk]
  v      ~ N(0,1) / sqrt(dk)                                            shape [B,H,T,dv]
  x      ~ N(0,1) (the gate's pre-activation)                           shape [B,H,T,dk]
  do     ~ N(0,1) / sqrt(dk)    drawn only when a backward is needed    shape [B,H,T,dv]

  g = logsigmoid(x) / 16, computed in float64 and stored as float32 (per token and per d_k
  channel, always <= 0: the log of a decay in (0, 1)).

q, k, v and do are then rounded to bfloat16 with round-to-nearest-even for the bf16 workloads
(torch's own cast) and kept in float32 for the fp32 ones.  The oracle sees exactly these rounded
values, widened to float64.

Gate variants for stress cases (same draw, different map from x to g):
  "logsigmoid16"  logsigmoid(x)/16 (the default; mean about -0.05 per token)
  "weak"          logsigmoid(x)/1024 (segments interact over thousands of tokens)
  "zero"          g = 0 (no decay at all)
  "strong"        -4 + 0.25*x clipped to <= 0 (about -4 per token: near the factorisation limit)
  "mixed"         even channels weak, odd channels strong
"""
from __future__ import annotations

import math
from dataclasses import dataclass, asdict

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    """One GLA problem instance: shapes, chunk size C, segment count P and scan block count K."""
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    P: int
    K: int
    dtype: str  # "bf16" or "f32" (q, k, v, do and o, dq, dk, dv); g, dg and states are fp32
    bwd: bool   # whether the workload includes the backward pass

    @property
    def L(self) -> int:
        return self.T // self.P

    def as_dict(self) -> dict:
        return asdict(self)


# The five workloads the method is exercised on.  Names say what they are.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32_t256_p4", B=1, H=1, T=256, dk=16, dv=16, chunk=16, P=4, K=2, dtype="f32", bwd=False),
        Workload("fwd_b2h4_t16k_p1", B=2, H=4, T=16384, dk=128, dv=256, chunk=64, P=1, K=1, dtype="bf16", bwd=False),
        Workload("fwd_h4_t32k_p8", B=1, H=4, T=32768, dk=128, dv=256, chunk=64, P=8, K=4, dtype="bf16", bwd=False),
        Workload("fwdbwd_h16_t16k_p4", B=1, H=16, T=16384, dk=128, dv=128, chunk=64, P=4, K=4, dtype="bf16", bwd=True),
        Workload("fwdbwd_h4_t1m_p64", B=1, H=4, T=1048576, dk=128, dv=256, chunk=64, P=64, K=8, dtype="bf16", bwd=True),
    ]
}

# The 16k-token-segment fwd+bwd workload: 64 segments of 16384 tokens, 4 heads.
HEADLINE = "fwdbwd_h4_t1m_p64"


def _logsigmoid64(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def gate_from_normal(x: np.ndarray, gate: str) -> np.ndarray:
    """Map the gate's standard-normal draw to float32 log-gates (all <= 0)."""
    if gate == "logsigmoid16":
        g = _logsigmoid64(x) / 16.0
    elif gate == "weak":
        g = _logsigmoid64(x) / 1024.0
    elif gate == "zero":
        g = np.zeros(x.shape, dtype=np.float64)
    elif gate == "strong":
        g = np.minimum(-4.0 + 0.25 * x.astype(np.float64), 0.0)
    elif gate == "mixed":
        g = _logsigmoid64(x) / 1024.0
        strong = np.minimum(-4.0 + 0.25 * x.astype(np.float64), 0.0)
        g[..., 1::2] = strong[..., 1::2]
    else:
        raise ValueError("unknown gate variant %r" % gate)
    return g.astype(np.float32)


def to_bf16_rne(x: np.ndarray) -> torch.Tensor:
    """float32 numpy -> bfloat16 torch tensor, round-to-nearest-even (torch's cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def generate(B: int, H: int, T: int, dk: int, dv: int, dtype: str = "bf16", seed: int = 0,
             bwd: bool = False, gate: str = "logsigmoid16") -> dict:
    """Draw one problem instance.  Returns CPU torch tensors q, k, v, g (and do if bwd).

    q, k, v, do are torch.bfloat16 (dtype="bf16") or torch.float32 (dtype="f32"); g is float32.
    """
    if dtype not in ("bf16", "f32"):
        raise ValueError("dtype must be 'bf16' or 'f32'")
    rng = np.random.default_rng(seed)
    s = np.float32(1.0 / math.sqrt(dk))
    out = {}
    for name, d in (("q", dk), ("k", dk), ("v", dv)):
        out[name] = rng.standard_normal((B, H, T, d), dtype=np.float32) * s
    x = rng.standard_normal((B, H, T, dk), dtype=np.float32)
    g = gate_from_normal(x, gate)
    del x
    if bwd:
        out["do"] = rng.standard_normal((B, H, T, dv), dtype=np.float32) * s
    res = {}
    for name, arr in out.items():
        res[name] = to_bf16_rne(arr) if dtype == "bf16" else torch.from_numpy(np.ascontiguousarray(arr))
    res["g"] = torch.from_numpy(g)
    return res


def generate_workload(w: Workload, seed: int = 0, gate: str = "logsigmoid16", bwd=None) -> dict:
    return generate(w.B, w.H, w.T, w.dk, w.dv, w.dtype, seed, w.bwd if bwd is None else bwd, gate)


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a (bf16 or fp32) tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)
