"""Seeded synthetic inputs for the GLA workloads (no method arithmetic lives here).

This module only draws random numbers and rounds them; the oracle and the HIP path both consume
its output and nothing else is shared between them.

Recipe.  Every (tensor, batch b, head h) slice [T, d] is cut into row blocks of 8192 tokens
(the last one may be shorter); block r has its own numpy generator
``default_rng(SeedSequence([seed, tensor_id, b, h, r]))`` drawing ``standard_normal(dtype=float32)``
in C order.  Blocks are therefore independent of each other and of the problem's B and H, are
drawn in parallel, and any single head can be regenerated on its own (``generate_head``):

  tensor_id 0  q   ~ N(0,1) / sqrt(dk)    scaled in float32                  [B,H,T,dk]
  tensor_id 1  k   ~ N(0,1) / sqrt(dk)                                       [B,H,T,dk]
  tensor_id 2  v   ~ N(0,1) / sqrt(dk)                                       [B,H,T,dv]
  tensor_id 3  x   ~ N(0,1), the gate's pre-activation                        [B,H,T,dk]
  tensor_id 4  do  ~ N(0,1) / sqrt(dk)    only when a backward is needed     [B,H,T,dv]

  g = logsigmoid(x) / 16, computed in float64 and stored as float32 (per token and per d_k
  channel, always <= 0: the log of a decay in (0, 1)).

q, k, v and do are then rounded to bfloat16 with round-to-nearest-even for the bf16 workloads
(bit arithmetic equal to torch's cast for finite values) and kept in float32 for the fp32 ones.  The oracle sees exactly these rounded
values, widened to float64.

Gate variants for stress cases (same draw, different map from x to g):
  "logsigmoid16"  logsigmoid(x)/16 (the default; mean about -0.05 per token)
  "weak"          logsigmoid(x)/1024 (segments interact over thousands of tokens)
  "zero"          g = 0 (no decay at all)
  "strong"        -2 + 0.25*x clipped to <= 0 (about -2 per token: -64 over a 32-token chunk)
  "strong5"       -5 + 0.25*x clipped to <= 0 (about -5 per token: -80 over 16 tokens, -320 over
                  a 64-token chunk; every chunk then runs the exact sub-block kernels)
  "mixed"         even channels weak, odd channels strong
  "scalar"        one decay per token and head (the LASP / TNL setting): logsigmoid(x[t, 0])/16 of
                  the token's first draw, the same for every d_k channel (the kernels are unchanged:
                  the gate is simply broadcast)
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
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
    x = np.asarray(x)
    if x.size > _BLOCK:  # stay in cache: the float64 temporaries are per block
        flat = x.reshape(-1)
        out = np.empty(flat.shape, dtype=np.float32)
        for i in range(0, flat.size, _BLOCK):
            out[i:i + _BLOCK] = gate_from_normal(flat[i:i + _BLOCK], gate)
        return out.reshape(x.shape)
    if gate == "logsigmoid16":
        g = _logsigmoid64(x) / 16.0
    elif gate == "weak":
        g = _logsigmoid64(x) / 1024.0
    elif gate == "zero":
        g = np.zeros(x.shape, dtype=np.float64)
    elif gate == "strong":
        g = np.minimum(-2.0 + 0.25 * x.astype(np.float64), 0.0)
    elif gate == "strong5":
        g = np.minimum(-5.0 + 0.25 * x.astype(np.float64), 0.0)
    elif gate == "mixed":
        g = _logsigmoid64(x) / 1024.0
        strong = np.minimum(-2.0 + 0.25 * x.astype(np.float64), 0.0)
        g[..., 1::2] = strong[..., 1::2]
    else:
        raise ValueError("unknown gate variant %r" % gate)
    return g.astype(np.float32)


_BLOCK = 1 << 16
_ROWS = 8192
_TENSORS = (("q", 0, "dk"), ("k", 1, "dk"), ("v", 2, "dv"), ("g", 3, "dk"), ("do", 4, "dv"))


def to_bf16_rne(x: np.ndarray) -> torch.Tensor:
    """float32 numpy -> bfloat16 torch tensor, round-to-nearest-even (torch's cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _bf16_bits(x: np.ndarray, out: np.ndarray):
    """Round finite float32 values to bfloat16 (nearest, ties to even); writes the uint16 bits."""
    u = x.view(np.uint32)
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u
    np.right_shift(r, 16, out=r)
    out[...] = r.astype(np.uint16)


def _fill(seed, tensor_id, b, h, r0, rows, d, scale, gate, bf16, out):
    rng = np.random.default_rng(np.random.SeedSequence([seed, tensor_id, b, h, r0 // _ROWS]))
    x = rng.standard_normal((rows, d), dtype=np.float32)
    if tensor_id == 3:
        if gate == "scalar":
            out[...] = gate_from_normal(x[:, :1], "logsigmoid16")
        else:
            out[...] = gate_from_normal(x, gate)
        return
    x *= scale
    if bf16:
        _bf16_bits(x, out)
    else:
        out[...] = x


def _draw(B, H, T, dk, dv, heads, seed, bwd, gate, dtype, threads):
    s = np.float32(1.0 / math.sqrt(dk))
    dims = {"dk": dk, "dv": dv}
    names = [t for t in _TENSORS if bwd or t[0] != "do"]
    bf16 = dtype == "bf16"
    arrays = {}
    for n, _, dd in names:
        dt = np.float32 if (n == "g" or not bf16) else np.uint16
        arrays[n] = np.empty((B, H, T, dims[dd]), dtype=dt)
    jobs = []
    for n, tid, _ in names:
        for bi, b in enumerate(heads[0]):
            for hi, h in enumerate(heads[1]):
                for r0 in range(0, T, _ROWS):
                    jobs.append((n, tid, bi, hi, b, h, r0, min(_ROWS, T - r0)))

    def run(j):
        n, tid, bi, hi, b, h, r0, rows = j
        out = arrays[n][bi, hi, r0:r0 + rows]
        _fill(seed, tid, b, h, r0, rows, out.shape[-1], s, gate, bf16 and n != "g", out)

    with ThreadPoolExecutor(max_workers=threads or min(16, os.cpu_count() or 4)) as ex:
        list(ex.map(run, jobs))
    res = {}
    for n, arr in arrays.items():
        t = torch.from_numpy(arr)
        res[n] = t.view(torch.bfloat16) if arr.dtype == np.uint16 else t
    return res


def generate(B: int, H: int, T: int, dk: int, dv: int, dtype: str = "bf16", seed: int = 0,
             bwd: bool = False, gate: str = "logsigmoid16", threads: int = 0) -> dict:
    """Draw one problem instance.  Returns CPU torch tensors q, k, v, g (and do if bwd).

    q, k, v, do are torch.bfloat16 (dtype="bf16") or torch.float32 (dtype="f32"); g is float32.
    """
    if dtype not in ("bf16", "f32"):
        raise ValueError("dtype must be 'bf16' or 'f32'")
    return _draw(B, H, T, dk, dv, (range(B), range(H)), seed, bwd, gate, dtype, threads)


def generate_head(B: int, H: int, T: int, dk: int, dv: int, b: int, h: int, dtype: str = "bf16",
                  seed: int = 0, bwd: bool = False, gate: str = "logsigmoid16", threads: int = 0) -> dict:
    """The (b, h) slice of ``generate(B, H, ...)``, shaped [1, 1, T, d], drawn on its own."""
    if not (0 <= b < B and 0 <= h < H):
        raise ValueError("head (%d, %d) outside B=%d, H=%d" % (b, h, B, H))
    return _draw(1, 1, T, dk, dv, ([b], [h]), seed, bwd, gate, dtype, threads)


def generate_workload(w: Workload, seed: int = 0, gate: str = "logsigmoid16", bwd=None) -> dict:
    return generate(w.B, w.H, w.T, w.dk, w.dv, w.dtype, seed, w.bwd if bwd is None else bwd, gate)


def add_strong_windows(g: torch.Tensor, P: int, n: int, length: int = 64, value: float = -3.0) -> torch.Tensor:
    """A copy of the log-gates g [B, H, T, dk] with n strongly decaying stretches: `length` tokens of
    g = `value` in every channel, in the middle of n of the B*H*P segments spread evenly over them
    (segment i * (B*H*P // n) for i < n, counted over b, h, then segment).  A stretch like this
    sends its segment's chunks past the fast kernels' decay bound."""
    B, H, T, _ = g.shape
    units, L = B * H * P, T // P
    if not 0 <= n <= units or length > L:
        raise ValueError("n must be in [0, B*H*P] and length at most the segment length")
    out = g.clone()
    for i in range(n):
        u = i * (units // n)
        b, r = divmod(u, H * P)
        h, p = divmod(r, P)
        t0 = p * L + (L - length) // 2
        out[b, h, t0:t0 + length] = value
    return out


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a (bf16 or fp32) tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)
