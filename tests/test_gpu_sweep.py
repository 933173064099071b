"""A seeded random sweep of configurations, fwd+bwd through every step, against the oracle.

Each case draws together:
- a compiled (dtype, d_k, d_v, chunk) instantiation;
- B <= 3, H <= 5, P <= 11 segments of 1..6 chunks, and a scan block count K;
- a gate recipe (the strong ones run the exact sub-block kernels);
- whether boundary states h0 and dh_T are given.

It runs 40 cases by default.  Set GLA_SWEEP to run more (GLA_SWEEP=2000 takes about four minutes
on one MI355X), and GLA_SWEEP_SEED to draw another sample.
"""
import os

import numpy as np
import pytest

from test_gpu_parity import SUPPORTED, run_case

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
