"""The oracle's pins are sharp: plant plausible mistakes in a copy of the C oracle and check that
one of the pins used in test_oracle.py rejects every one of them.

Each mutant is a textual edit of gla_oracle.c compiled into a temporary library (on the CPU).
The pins used here are the quadratic closed form (forward) and torch float64 autograd through an
independent torch rendering of that form (backward).
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from test_oracle import _case, _rel, _torch_quadratic

SRC = os.path.join(os.path.dirname(oracle.__file__), "gla_oracle.c")

FWD_MUTANTS = {
    "gate_applied_after_adding_kv": (
        "S[c * JB + jj] = a * S[c * JB + jj] + ktc * vb[(long)t * dv + j0 + jj];",
        "S[c * JB + jj] = a * (S[c * JB + jj] + ktc * vb[(long)t * dv + j0 + jj]);"),
    "output_reads_state_before_update": (
        "            S[c * JB + jj] = a * S[c * JB + jj] + ktc * vb[(long)t * dv + j0 + jj];\n"
        "            acc[jj] += qtc * S[c * JB + jj];",
        "            acc[jj] += qtc * S[c * JB + jj];\n"
        "            S[c * JB + jj] = a * S[c * JB + jj] + ktc * vb[(long)t * dv + j0 + jj];"),
    "gate_sign_flipped": (
        "          const double a = exp(gb[(long)t * dk + c]);\n          const double ktc",
        "          const double a = exp(-gb[(long)t * dk + c]);\n          const double ktc"),
    "initial_state_dropped": (
        "S[c * JB + jj] = h0 ? h0[bh * (long)dk * dv + (long)c * dv + j0 + jj] : 0.0;",
        "S[c * JB + jj] = 0.0;"),
    "query_of_previous_token": (
        "          const double qtc = qb[(long)t * dk + c];\n          for (int jj = 0; jj < nj; ++jj) {\n"
        "            S[c * JB",
        "          const double qtc = qb[(long)(t > 0 ? t - 1 : 0) * dk + c];\n"
        "          for (int jj = 0; jj < nj; ++jj) {\n            S[c * JB"),
}

BWD_MUTANTS = {
    "dq_reads_state_before_update": (
        "          S[j] = a * S[j] + ktc * vb[(long)t * dv + j];\n"
        "          acc += S[j] * db[(long)t * dv + j];",
        "          acc += S[j] * db[(long)t * dv + j];\n"
        "          S[j] = a * S[j] + ktc * vb[(long)t * dv + j];"),
    "dk_decay_applied_one_token_late": (
        "          U[j] += qtc * db[(long)t * dv + j];\n          acc += U[j] * vb[(long)t * dv + j];",
        "          U[j] = exp(gb[(long)t * dk + c]) * U[j] + qtc * db[(long)t * dv + j];\n"
        "          acc += U[j] * vb[(long)t * dv + j];"),
    "dv_query_term_sign": (
        "U[c * JB + jj] += qtc * db[(long)t * dv + j0 + jj];",
        "U[c * JB + jj] -= qtc * db[(long)t * dv + j0 + jj];"),
    "dg_final_state_term_dropped": (
        "double run = dg_const[u];",
        "double run = 0.0 * dg_const[u];"),
    "dg_key_term_sign": (
        "run += q[i] * dq[i] - k[i] * dkk[i];",
        "run += q[i] * dq[i] + k[i] * dkk[i];"),
    "dh0_missing_first_gate": (
        "for (int j = 0; j < dv; ++j) dh0[bh * (long)dk * dv + (long)c * dv + j] = U[j];",
        "for (int j = 0; j < dv; ++j) dh0[bh * (long)dk * dv + (long)c * dv + j] = U[j] / exp(gb[c]);"),
}


def _build(tmp_path, name, edit):
    src = open(SRC).read()
    if edit is not None:
        old, new = edit
        assert src.count(old) >= 1, "mutation site not found: %s" % name
        src = src.replace(old, new, 1)
    cpath = tmp_path / ("%s.c" % name)
    cpath.write_text(src)
    so = tmp_path / ("%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", str(so), str(cpath), "-lm"], check=True)
    return oracle.load_library(str(so))


def _fwd_pin_error():
    c = _case(1, 2, 23, 5, 3, seed=28, with_h0=True)
    o, _ = oracle.gla_fwd(c["q"], c["k"], c["v"], c["g"], c["h0"])
    return _rel(o, oracle.bruteforce_fwd(c["q"], c["k"], c["v"], c["g"], c["h0"]))


def _bwd_pin_error():
    c = _case(1, 2, 13, 5, 4, seed=8, gscale=0.4, with_h0=True, with_do=True)
    ts = {n: torch.tensor(c[n], dtype=torch.float64, requires_grad=n in ("q", "k", "v", "g", "h0"))
          for n in ("q", "k", "v", "g", "h0", "do", "dhT")}
    _torch_quadratic(ts["q"], ts["k"], ts["v"], ts["g"], ts["h0"], ts["do"], ts["dhT"]).backward()
    gr = oracle.gla_bwd(c["q"], c["k"], c["v"], c["g"], c["do"], c["h0"], c["dhT"])
    return max(_rel(gr[d], ts[x].grad.numpy())
               for x, d in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("h0", "dh0")])


def test_unmutated_copy_passes_both_pins(tmp_path, monkeypatch):
    monkeypatch.setattr(oracle, "_lib", _build(tmp_path, "clean", None))
    assert _fwd_pin_error() < 1e-13
    assert _bwd_pin_error() < 1e-12


@pytest.mark.parametrize("name", sorted(FWD_MUTANTS))
def test_forward_pin_rejects_mutant(tmp_path, monkeypatch, name):
    monkeypatch.setattr(oracle, "_lib", _build(tmp_path, name, FWD_MUTANTS[name]))
    assert _fwd_pin_error() > 1e-3


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_pin_rejects_mutant(tmp_path, monkeypatch, name):
    monkeypatch.setattr(oracle, "_lib", _build(tmp_path, name, BWD_MUTANTS[name]))
    assert _bwd_pin_error() > 1e-3
