"""Pins for the float64 oracle: every check here compares it with something other than itself.

* the quadratic closed form (explicit sum over token pairs and channels, numpy)
* textbook special cases: no decay is causal linear attention (QK^T masked) V, a full decay
  leaves only the token's own term, a single token is (q.k) v
* finite differences of the forward for every gradient, and torch float64 autograd through an
  independent torch rendering of the quadratic form
* the direct form of dg against the closed form the oracle uses
* homogeneity of o in q, k and v (sum <dq,q> = sum <dk,k> = sum <dv,v> = sum <do,o>)
* ZeCO's decomposition (local pass, decay-and-add scan, correction) against the plain recurrence,
  for the forward and the backward, and the scan's special cases (no decay: exclusive prefix sum;
  full decay: a shift)
"""
import numpy as np
import pytest
import torch

import oracle


def _case(B=1, H=2, T=23, dk=5, dv=3, seed=0, gscale=0.3, with_h0=False, with_do=False):
    rng = np.random.default_rng(seed)
    d = {
        "q": rng.standard_normal((B, H, T, dk)),
        "k": rng.standard_normal((B, H, T, dk)),
        "v": rng.standard_normal((B, H, T, dv)),
        # log-gates <= 0 with a spread of per-channel decays
        "g": -np.abs(rng.standard_normal((B, H, T, dk))) * gscale,
    }
    if with_h0:
        d["h0"] = rng.standard_normal((B, H, dk, dv))
    if with_do:
        d["do"] = rng.standard_normal((B, H, T, dv))
        d["dhT"] = rng.standard_normal((B, H, dk, dv))
    return d


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ------------------------------------------------------------------------------------------ fwd

@pytest.mark.parametrize("shape", [(1, 2, 23, 5, 3), (2, 1, 1, 4, 6), (1, 1, 17, 1, 2), (1, 3, 40, 8, 8)])
@pytest.mark.parametrize("with_h0", [False, True])
def test_fwd_matches_quadratic_form(shape, with_h0):
    B, H, T, dk, dv = shape
    c = _case(B, H, T, dk, dv, seed=T + dk, with_h0=with_h0)
    o, hT = oracle.gla_fwd(c["q"], c["k"], c["v"], c["g"], c.get("h0"))
    ref = oracle.bruteforce_fwd(c["q"], c["k"], c["v"], c["g"], c.get("h0"))
    assert _rel(o, ref) < 1e-13
    # end state from its own closed form: sum_s exp(B_T - B_s) k_s v_s^T + exp(B_T) h0
    Bc = np.cumsum(c["g"], axis=2)
    w = np.exp(Bc[:, :, -1:, :] - Bc)
    S = np.einsum("bhsc,bhsj->bhcj", c["k"] * w, c["v"])
    if with_h0:
        S = S + np.exp(Bc[:, :, -1, :])[..., None] * c["h0"]
    assert _rel(hT, S) < 1e-13


def test_fwd_without_decay_is_masked_linear_attention():
    c = _case(1, 2, 31, 6, 4, seed=3, with_h0=True)
    g0 = np.zeros_like(c["g"])
    o, hT = oracle.gla_fwd(c["q"], c["k"], c["v"], g0, c["h0"])
    A = np.tril(np.einsum("bhtc,bhsc->bhts", c["q"], c["k"]))
    ref = np.einsum("bhts,bhsj->bhtj", A, c["v"]) + np.einsum("bhtc,bhcj->bhtj", c["q"], c["h0"])
    assert _rel(o, ref) < 1e-13
    assert _rel(hT, np.einsum("bhsc,bhsj->bhcj", c["k"], c["v"]) + c["h0"]) < 1e-13


def test_fwd_full_decay_keeps_only_own_token():
    c = _case(1, 2, 19, 5, 3, seed=4, with_h0=True)
    gfull = np.full_like(c["g"], -1e4)  # exp underflows to exactly 0 in float64
    o, hT = oracle.gla_fwd(c["q"], c["k"], c["v"], gfull, c["h0"])
    ref = np.einsum("bhtc,bhtc->bht", c["q"], c["k"])[..., None] * c["v"]
    assert _rel(o, ref) < 1e-14
    assert _rel(hT, np.einsum("bhc,bhj->bhcj", c["k"][:, :, -1], c["v"][:, :, -1])) < 1e-14


def test_fwd_single_token():
    c = _case(2, 2, 1, 4, 3, seed=5, with_h0=True)
    o, _ = oracle.gla_fwd(c["q"], c["k"], c["v"], c["g"], c["h0"])
    a = np.exp(c["g"][:, :, 0, :])
    ref = (np.einsum("bhc,bhc->bh", c["q"][:, :, 0], c["k"][:, :, 0])[..., None] * c["v"][:, :, 0]
           + np.einsum("bhc,bhcj->bhj", c["q"][:, :, 0] * a, c["h0"]))
    assert _rel(o[:, :, 0], ref) < 1e-14


def test_fwd_thread_count_does_not_change_bits():
    c = _case(1, 3, 64, 8, 12, seed=6, with_h0=True)
    o1, h1 = oracle.gla_fwd(c["q"], c["k"], c["v"], c["g"], c["h0"], threads=1)
    o4, h4 = oracle.gla_fwd(c["q"], c["k"], c["v"], c["g"], c["h0"], threads=4)
    assert np.array_equal(o1, o4) and np.array_equal(h1, h4)


# ------------------------------------------------------------------------------------------ bwd

def _loss(c, **over):
    d = dict(c)
    d.update(over)
    o, hT = oracle.gla_fwd(d["q"], d["k"], d["v"], d["g"], d.get("h0"))
    return float(np.sum(o * d["do"]) + np.sum(hT * d["dhT"]))


@pytest.mark.parametrize("with_h0", [False, True])
def test_bwd_matches_finite_differences(with_h0):
    c = _case(1, 2, 11, 4, 3, seed=7, gscale=0.5, with_h0=with_h0, with_do=True)
    grads = oracle.gla_bwd(c["q"], c["k"], c["v"], c["g"], c["do"], c.get("h0"), c["dhT"])
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg")] + ([("h0", "dh0")] if with_h0 else [])
    eps = 1e-6
    rng = np.random.default_rng(0)
    for x, dx in names:
        base = c[x]
        idxs = [tuple(rng.integers(0, s) for s in base.shape) for _ in range(12)]
        for idx in idxs:
            p = base.copy()
            m = base.copy()
            p[idx] += eps
            m[idx] -= eps
            fd = (_loss(c, **{x: p}) - _loss(c, **{x: m})) / (2 * eps)
            an = grads[dx][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (x, idx, fd, an)


def _torch_quadratic(q, k, v, g, h0, do, dhT):
    """Independent torch rendering of the unrolled recurrence (float64), for autograd."""
    Bc = torch.cumsum(g, dim=2)
    T = q.shape[2]
    outs = []
    for t in range(T):
        w = torch.exp(Bc[:, :, t:t + 1, :] - Bc[:, :, : t + 1, :])
        coef = (q[:, :, t:t + 1, :] * k[:, :, : t + 1, :] * w).sum(-1)  # [B,H,t+1]
        ot = (coef.unsqueeze(-1) * v[:, :, : t + 1, :]).sum(2)
        ot = ot + ((q[:, :, t, :] * torch.exp(Bc[:, :, t, :])).unsqueeze(-1) * h0).sum(2)
        outs.append(ot)
    o = torch.stack(outs, dim=2)
    wT = torch.exp(Bc[:, :, -1:, :] - Bc)
    ST = ((k * wT).unsqueeze(-1) * v.unsqueeze(-2)).sum(2) + torch.exp(Bc[:, :, -1, :]).unsqueeze(-1) * h0
    return (o * do).sum() + (ST * dhT).sum()


def test_bwd_matches_torch_autograd():
    c = _case(2, 2, 13, 5, 4, seed=8, gscale=0.4, with_h0=True, with_do=True)
    ts = {n: torch.tensor(c[n], dtype=torch.float64, requires_grad=n in ("q", "k", "v", "g", "h0"))
          for n in ("q", "k", "v", "g", "h0", "do", "dhT")}
    L = _torch_quadratic(ts["q"], ts["k"], ts["v"], ts["g"], ts["h0"], ts["do"], ts["dhT"])
    L.backward()
    grads = oracle.gla_bwd(c["q"], c["k"], c["v"], c["g"], c["do"], c["h0"], c["dhT"])
    for x, dx in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("h0", "dh0")]:
        assert _rel(grads[dx], ts[x].grad.numpy()) < 1e-12, x


def test_dg_closed_form_matches_direct_form():
    c = _case(1, 3, 29, 6, 5, seed=9, gscale=0.6, with_h0=True, with_do=True)
    grads = oracle.gla_bwd(c["q"], c["k"], c["v"], c["g"], c["do"], c["h0"], c["dhT"])
    direct = oracle.gla_dg_direct(c["q"], c["k"], c["v"], c["g"], c["do"], c["h0"], c["dhT"])
    assert _rel(grads["dg"], direct) < 1e-12


def test_homogeneity_identity():
    c = _case(1, 2, 37, 6, 5, seed=10, with_do=True)
    o, _ = oracle.gla_fwd(c["q"], c["k"], c["v"], c["g"])
    gr = oracle.gla_bwd(c["q"], c["k"], c["v"], c["g"], c["do"])
    ref = np.sum(c["do"] * o, axis=(2, 3))
    for x, dx in [("q", "dq"), ("k", "dk"), ("v", "dv")]:
        got = np.sum(c[x] * gr[dx], axis=(2, 3))
        assert np.max(np.abs(got - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref))), x


def test_bwd_thread_count_does_not_change_bits():
    c = _case(1, 2, 33, 7, 9, seed=11, with_h0=True, with_do=True)
    a = oracle.gla_bwd(c["q"], c["k"], c["v"], c["g"], c["do"], c["h0"], c["dhT"], threads=1)
    b = oracle.gla_bwd(c["q"], c["k"], c["v"], c["g"], c["do"], c["h0"], c["dhT"], threads=3)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


# ------------------------------------------------------------------------------- decomposition

@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("with_h0", [False, True])
def test_segmented_forward_equals_plain_recurrence(P, with_h0):
    # weak decay so that every segment still sees the earlier ones
    c = _case(2, 2, 64, 6, 5, seed=12 + P, gscale=0.02, with_h0=with_h0)
    o, hT = oracle.gla_fwd(c["q"], c["k"], c["v"], c["g"], c.get("h0"))
    z = oracle.zeco_fwd(c["q"], c["k"], c["v"], c["g"], P, c.get("h0"))
    assert _rel(z["o"], o) < 1e-12
    assert _rel(z["h_final"], hT) < 1e-12
    # the state entering each segment is the plain recurrence's state after the prefix
    L = 64 // P
    for p in range(P):
        if p == 0:
            ref = c["h0"] if with_h0 else np.zeros_like(z["S_in"][:, :, 0])
        else:
            _, ref = oracle.gla_fwd(c["q"][:, :, : p * L], c["k"][:, :, : p * L], c["v"][:, :, : p * L],
                                    c["g"][:, :, : p * L], c.get("h0"))
        assert np.max(np.abs(z["S_in"][:, :, p] - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))
    # the local pass is the plain recurrence of each segment on its own, from zero
    if P > 1:
        o1, h1 = oracle.gla_fwd(c["q"][:, :, L:2 * L], c["k"][:, :, L:2 * L], c["v"][:, :, L:2 * L],
                                c["g"][:, :, L:2 * L])
        assert np.array_equal(z["o_local"][:, :, L:2 * L], o1)
        assert np.array_equal(z["S_local"][:, :, 1], h1)


@pytest.mark.parametrize("P", [1, 3, 4])
@pytest.mark.parametrize("with_ends", [False, True])
def test_segmented_backward_equals_plain_recurrence(P, with_ends):
    c = _case(1, 2, 48, 5, 4, seed=20 + P, gscale=0.02, with_h0=with_ends, with_do=True)
    dhT = c["dhT"] if with_ends else None
    ref = oracle.gla_bwd(c["q"], c["k"], c["v"], c["g"], c["do"], c.get("h0"), dhT)
    z = oracle.zeco_fwd(c["q"], c["k"], c["v"], c["g"], P, c.get("h0"))
    b = oracle.zeco_bwd(c["q"], c["k"], c["v"], c["g"], c["do"], P, z["S_in"], z["logdecay"],
                        z["h_final"], dhT)
    for n in ("dq", "dk", "dv", "dg"):
        assert _rel(b[n], ref[n]) < 1e-11, n
    assert _rel(b["dh0"], ref["dh0"]) < 1e-11


def test_segmented_backward_with_strong_decay_is_local():
    # with a strong decay no gradient crosses a segment boundary: the corrections vanish
    c = _case(1, 1, 32, 4, 3, seed=30, gscale=0.0, with_do=True)
    g = np.full_like(c["g"], -60.0)
    z = oracle.zeco_fwd(c["q"], c["k"], c["v"], g, 4)
    b = oracle.zeco_bwd(c["q"], c["k"], c["v"], g, c["do"], 4, z["S_in"], z["logdecay"], z["h_final"])
    assert np.allclose(b["dk"], b["dk_local"], rtol=0, atol=1e-20)
    assert np.allclose(b["dv"], b["dv_local"], rtol=0, atol=1e-20)


def test_scan_without_decay_is_exclusive_prefix_sum():
    rng = np.random.default_rng(40)
    S = rng.standard_normal((2, 3, 6, 4, 5))
    h0 = rng.standard_normal((2, 3, 4, 5))
    ld = np.zeros((2, 3, 6, 4))
    carry, hout = oracle.segment_scan(S, ld, h0)
    ex = np.concatenate([np.zeros_like(S[:, :, :1]), np.cumsum(S, axis=2)[:, :, :-1]], axis=2) + h0[:, :, None]
    assert _rel(carry, ex) < 1e-14
    assert _rel(hout, S.sum(axis=2) + h0) < 1e-14
    # reverse: carry[p] = dhT + sum of D over the later segments
    carry_r, dh0 = oracle.segment_scan(S, ld, h0, reverse=True)
    suffix = np.flip(np.cumsum(np.flip(S, axis=2), axis=2), axis=2)
    ex_r = np.concatenate([suffix[:, :, 1:], np.zeros_like(S[:, :, :1])], axis=2) + h0[:, :, None]
    assert _rel(carry_r, ex_r) < 1e-14
    assert _rel(dh0, S.sum(axis=2) + h0) < 1e-14


def test_scan_with_full_decay_is_a_shift():
    rng = np.random.default_rng(41)
    S = rng.standard_normal((1, 2, 5, 3, 4))
    ld = np.full((1, 2, 5, 3), -1e4)
    carry, hout = oracle.segment_scan(S, ld, rng.standard_normal((1, 2, 3, 4)))
    assert np.array_equal(carry[:, :, 1:], S[:, :, :-1])
    assert np.array_equal(hout, S[:, :, -1])
    carry_r, dh0 = oracle.segment_scan(S, ld, None, reverse=True)
    assert np.array_equal(carry_r[:, :, :-1], S[:, :, 1:])
    assert np.array_equal(dh0, S[:, :, 0])


def test_scan_rows_are_independent():
    # the decay scales whole d_k rows: scanning a subset of rows gives those rows of the full scan
    rng = np.random.default_rng(42)
    S = rng.standard_normal((1, 2, 7, 8, 3))
    ld = -np.abs(rng.standard_normal((1, 2, 7, 8)))
    full, _ = oracle.segment_scan(S, ld, None)
    part, _ = oracle.segment_scan(S[:, :, :, 2:6], ld[:, :, :, 2:6], None)
    assert np.array_equal(full[:, :, :, 2:6], part)


@pytest.mark.parametrize("P,C", [(1, 4), (2, 8), (4, 4)])
def test_chunk_states_local_and_corrected(P, C):
    # the recorded states are the plain recurrence's state after every C tokens (prefix runs),
    # locally per segment and, after the correction step, globally
    c = _case(1, 2, 32, 4, 3, seed=50 + P, gscale=0.05, with_h0=True)
    z = oracle.zeco_fwd(c["q"], c["k"], c["v"], c["g"], P, c["h0"], chunk=C)
    L = 32 // P
    for n in range(32 // C):
        t1 = (n + 1) * C
        _, ref = oracle.gla_fwd(c["q"][:, :, :t1], c["k"][:, :, :t1], c["v"][:, :, :t1], c["g"][:, :, :t1], c["h0"])
        assert _rel(z["chunk_states"][:, :, n], ref) < 1e-12
        p0 = (t1 - 1) // L * L  # first token of this chunk's segment
        _, loc = oracle.gla_fwd(c["q"][:, :, p0:t1], c["k"][:, :, p0:t1], c["v"][:, :, p0:t1], c["g"][:, :, p0:t1])
        assert _rel(z["chunk_states_local"][:, :, n], loc) < 1e-12


# ------------------------------------------------------- the state passes' unrolled weighted sums

@pytest.mark.parametrize("gscale", [0.05, 3.0])
def test_segment_state_and_gradient_are_unrolled_weighted_sums(gscale):
    """The oracle's per-segment local state and state gradient against the recurrence unrolled:
    from S_t = diag(e^{g_t}) S_{t-1} + k_t v_t^T and a zero start, a segment's end state is
    sum_t exp(x_t) k_t v_t^T with x_t the log-gates after t in the segment, and the gradient
    w.r.t. the state entering it from its own outputs (o_t = S_t^T q_t) is sum_t exp(a_t) q_t do_t^T
    with a_t the log-gates from the segment's start through t.  These are the sums the state
    passes add chunk by chunk from the far end.  With strong decay (gscale 3: about -2.4 per token)
    the tokens whose weight is below e^-112 in every channel, which the passes leave out, move
    neither sum by more than 1e-40 of its size."""
    P, T = 2, 256
    c = _case(1, 2, T, 4, 3, seed=77, gscale=gscale, with_do=True)
    z = oracle.zeco_fwd(c["q"], c["k"], c["v"], c["g"], P)
    b = oracle.zeco_bwd(c["q"], c["k"], c["v"], c["g"], c["do"], P, z["S_in"], z["logdecay"])
    L = T // P
    for p in range(P):
        q, k, v, g, do = (c[n][:, :, p * L:(p + 1) * L] for n in ("q", "k", "v", "g", "do"))
        after = np.cumsum(g[:, :, ::-1], axis=2)[:, :, ::-1] - g  # sum over tau > t
        through = np.cumsum(g, axis=2)                              # sum over tau <= t
        S = np.einsum("bhtc,bhtj->bhcj", k * np.exp(after), v)
        D = np.einsum("bhtc,bhtj->bhcj", q * np.exp(through), do)
        assert _rel(z["S_local"][:, :, p], S) < 1e-12
        assert _rel(b["D_local"][:, :, p], D) < 1e-12
        assert np.allclose(z["logdecay"][:, :, p], g.sum(axis=2), rtol=1e-12, atol=1e-12)
        keep_s = (after >= -112).any(axis=3, keepdims=True)   # [B, H, L, 1]: some channel above the cut
        keep_d = (through >= -112).any(axis=3, keepdims=True)
        S_cut = np.einsum("bhtc,bhtj->bhcj", k * np.exp(after) * keep_s, v)
        D_cut = np.einsum("bhtc,bhtj->bhcj", q * np.exp(through) * keep_d, do)
        assert _rel(S_cut, S) <= 1e-40 and _rel(D_cut, D) <= 1e-40
        if gscale > 1:  # the cut is reached inside the segment, from both ends
            assert not keep_s.all() and not keep_d.all()
