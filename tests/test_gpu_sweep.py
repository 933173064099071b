"""A seeded random sweep of configurations, fwd+bwd through every step, against the oracle.

Each case draws together:
- a compiled (dtype, d_k, d_v, chunk) instantiation;
- B <= 3, H <= 5, P <= 11 segments of 1..6 chunks, and a scan block count K;
- a gate recipe (the strong ones run the exact sub-block kernels);
- whether boundary states h0 and dh_T are given.

It runs 40 cases by default.  Set GLA_SWEEP to run more (GLA_SWEEP=2000 takes about four minutes
on one MI355X), and GLA_SWEEP_SEED to draw another sample.

A second sweep (test_random_strong_windows, GLA_SWEEP_WINDOWS cases, 10 by default) puts strongly
decaying stretches at random places into shapes with at least 256 units of 4 or more chunks, where
the flagged units are cut into pieces (the re-split) or, beyond the slots, run whole.

A third (test_random_configuration_states_first, GLA_SWEEP_SF cases, 24 by default) draws from the
same distribution and runs the order with the incoming states first: state passes that stop where
the decay ends, the scans, and the local passes from the true incoming states.
"""
import os

import numpy as np
import pytest
import torch

from sequence_state_scan_amd import gla, inputs
from test_gpu_parity import (SF_BWD_KEYS, SF_FWD_KEYS, SUPPORTED, TOL, FWD_KEYS, BWD_KEYS, check, dev, gpu_pipeline,
                             oracle_pipeline, reach_clamped, run_case, states_first_pipeline)

pytestmark = pytest.mark.gpu

N = int(os.environ.get("GLA_SWEEP", "40"))
SEED = int(os.environ.get("GLA_SWEEP_SEED", "7777"))
GATES = ("logsigmoid16", "weak", "strong", "scalar", "zero", "mixed", "strong5")


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype, dk, dv, chunk = SUPPORTED[int(rng.integers(len(SUPPORTED)))]
        B, H, P = int(rng.integers(1, 4)), int(rng.integers(1, 6)), int(rng.integers(1, 12))
        per_seg = int(rng.integers(1, 7))
        K = [k for k in (1, 2, 4, 8, 16) if dk % k == 0][int(rng.integers(0, 3))]
        gate = GATES[int(rng.integers(len(GATES)))]
        out.append((B, H, P * per_seg * chunk, dk, dv, chunk, P, K, dtype, gate, int(rng.integers(1000)),
                    bool(rng.integers(2))))
    return out


@pytest.mark.parametrize("case", _cases(N, SEED))
def test_random_configuration(case):
    B, H, T, dk, dv, chunk, P, K, dtype, gate, seed, carry = case
    run_case(B, H, T, dk, dv, chunk, P, K, dtype, bwd=True, gate=gate, seed=seed, carry=carry)


def _window_cases(n, seed):
    """Shapes with at least 256 units of 4 to 16 chunks (so flagged units are re-split), and 1 to 12
    strongly decaying stretches at random places: (b, h, first token, length, channel step, g)."""
    rng = np.random.default_rng(seed)
    fast = [c for c in SUPPORTED if c[3] != 16 or c[0] == "f32"]
    out = []
    while len(out) < n:
        dtype, dk, dv, chunk = fast[int(rng.integers(len(fast)))]
        if dk * dv > 64 * 128:
            continue
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 5))
        P = int(-(-256 // (B * H)))
        P += int(rng.integers(0, 2)) * P  # up to twice as many units as slots
        per_seg = (4, 8, 16)[int(rng.integers(3))]
        T = P * per_seg * chunk
        if B * H * T > 400_000:
            continue
        wins = []
        for _ in range(int(rng.integers(1, 13))):
            ln = int(rng.integers(8, 81))
            wins.append((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(T - ln)), ln,
                         int(rng.integers(1, 4)), -float(rng.uniform(2.0, 6.0))))
        out.append((dtype, B, H, T, dk, dv, chunk, P, wins, int(rng.integers(1000)), bool(rng.integers(2))))
    return out


@pytest.mark.parametrize("case", _window_cases(int(os.environ.get("GLA_SWEEP_WINDOWS", "10")), SEED + 1))
def test_random_strong_windows(case):
    """Strongly decaying stretches at random places: the units they touch are flagged and re-split
    (or, past the slots, run whole), the rest take the fast kernels; fwd+bwd against the oracle."""
    dtype, B, H, T, dk, dv, chunk, P, wins, seed, carry = case
    print("windows case", dtype, B, H, T, dk, dv, chunk, P, len(wins), flush=True)
    d = inputs.generate(B, H, T, dk, dv, dtype, seed, True, "logsigmoid16")
    g = d["g"].clone()
    for b, h, t0, ln, step, val in wins:
        g[b, h, t0:t0 + ln, ::step] = val
    d["g"] = g
    h0 = dhT = None
    if carry:
        rng = np.random.default_rng(seed + 100)
        h0 = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3)
        dhT = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3)
    gpu = gpu_pipeline(dev(d), chunk, P, 1, True, None if h0 is None else h0.cuda(),
                       None if dhT is None else dhT.cuda())
    ref = oracle_pipeline(d, chunk, P, True, None if h0 is None else h0.numpy(), None if dhT is None else dhT.numpy())
    check(gpu, ref, FWD_KEYS + BWD_KEYS, TOL[dtype], "windows %s B%d H%d T%d dk%d dv%d C%d P%d" %
          (dtype, B, H, T, dk, dv, chunk, P))


def _sf_runs(case):
    """bf16 chunk 16 has no state-pass kernel of its own: its state passes run in 32- or 64-token
    chunks, so the segments must hold whole ones."""
    B, H, T, dk, dv, chunk, P, K, dtype, gate, seed, carry = case
    return not (dtype == "bf16" and chunk == 16 and (T // P) % 32)


@pytest.mark.parametrize("case", [c for c in _cases(int(os.environ.get("GLA_SWEEP_SF", "24")), SEED + 2)
                                  if _sf_runs(c)])
def test_random_configuration_states_first(case):
    B, H, T, dk, dv, chunk, P, K, dtype, gate, seed, carry = case
    d = inputs.generate(B, H, T, dk, dv, dtype, seed, True, gate)
    h0 = dhT = None
    if carry:
        rng = np.random.default_rng(seed + 100)
        h0 = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3)
        dhT = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3)
    gpu = states_first_pipeline(dev(d), chunk, P, K, None if h0 is None else h0.cuda(),
                                None if dhT is None else dhT.cuda())
    ref = oracle_pipeline(d, chunk, P, True, None if h0 is None else h0.numpy(), None if dhT is None else dhT.numpy())
    check(reach_clamped(gpu), reach_clamped(ref), SF_FWD_KEYS + SF_BWD_KEYS, TOL[dtype],
          "states first B%d H%d T%d dk%d dv%d C%d P%d K%d %s %s" % (B, H, T, dk, dv, chunk, P, K, dtype, gate))
