"""GPU parity: every entry point of libgla.so, called through the C ABI (ctypes binding), against
the float64 oracle on the same seeded inputs.

Tolerance (per tensor): max|gpu - oracle| / max|oracle| <= 2e-2 for bf16 inputs, 1e-4 for fp32.
Intermediates (local outputs and states, segment carries, local gradients) are checked as well
as the final results, so a wrong step cannot hide behind a later one.
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle
from sequence_state_scan_amd import gla, inputs
from sequence_state_scan_amd.inputs import as_f64

pytestmark = pytest.mark.gpu
TOL = {"bf16": 2e-2, "f32": 1e-4}
FWD_KEYS = ("o_local", "cs_local", "S_local", "logdecay", "S_in", "h_final", "o", "cs")
BWD_KEYS = ("dq", "dk_local", "dv_local", "dg_local", "D_local", "G", "dh0", "dk", "dv", "dg")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def maxrel(x, r):
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = np.max(np.abs(r)) if r.size else 0.0
    num = np.max(np.abs(x - r)) if r.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def elemrel(x, r):
    """Element-wise relative error with a floor: max_i |x_i - r_i| / (|r_i| + 1e-3 max|r|).  Unlike
    maxrel it does not let a local error hide where the tensor is small (reported, not gated)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if not r.size:
        return 0.0
    floor = 1e-3 * np.max(np.abs(r))
    if floor == 0.0:
        return float(np.max(np.abs(x - r)))
    return float(np.max(np.abs(x - r) / (np.abs(r) + floor)))


def dev(d):
    return {k: v.to("cuda") for k, v in d.items()}


def gpu_pipeline(d, chunk, P, K, bwd, h0=None, dhT=None, ws=None):
    """Every step through the C ABI, keeping the intermediates.  Returns float64 numpy arrays.
    ws: the workspace of both chunked calls (default: the size for the fastest schedule)."""
    q, k, v, g = d["q"], d["k"], d["v"], d["g"]
    o, cs, S_loc, ld = gla.gla_chunk_fwd(q, k, v, g, chunk, P, workspace=ws)
    res = {"o_local": o.clone(), "cs_local": gla.chunk_states_dense(cs), "S_local": S_loc, "logdecay": ld}
    S_in, h_final = gla.gla_segment_scan(S_loc, ld, K, h_boundary=h0)
    gla.gla_segment_correct(gla.GLA_FWD, chunk, P, q=q, g=g, seg_in=S_in, o=o, chunk_states=cs)
    res.update(S_in=S_in, h_final=h_final, o=o, cs=gla.chunk_states_dense(cs))
    if bwd:
        dq, dk, dv, dg, D = gla.gla_chunk_bwd(q, k, v, g, d["do"], cs, S_in, chunk, P, workspace=ws)
        res.update(dq=dq, dk_local=dk.clone(), dv_local=dv.clone(), dg_local=dg.clone(), D_local=D)
        G, dh0 = gla.gla_segment_scan(D, ld, K, h_boundary=dhT, reverse=True)
        gla.gla_segment_correct(gla.GLA_BWD, chunk, P, k=k, v=v, g=g, seg_in=S_in, seg_grad=G,
                                chunk_states=cs, dk=dk, dv=dv, dg=dg)
        res.update(G=G, dh0=dh0, dk=dk, dv=dv, dg=dg)
    torch.cuda.synchronize()
    return {n: as_f64(t) for n, t in res.items()}


def oracle_pipeline(d, chunk, P, bwd, h0=None, dhT=None):
    a = {n: as_f64(t) for n, t in d.items()}
    z = oracle.zeco_fwd(a["q"], a["k"], a["v"], a["g"], P, h0, chunk=chunk)
    res = {"o_local": z["o_local"], "cs_local": z["chunk_states_local"], "S_local": z["S_local"],
           "logdecay": z["logdecay"], "S_in": z["S_in"], "h_final": z["h_final"], "o": z["o"],
           "cs": z["chunk_states"]}
    if bwd:
        b = oracle.zeco_bwd(a["q"], a["k"], a["v"], a["g"], a["do"], P, z["S_in"], z["logdecay"], z["h_final"], dhT)
        for n in BWD_KEYS:
            res[n] = b[n]
    return res


def homogeneity(x, dx, ref):
    """Per (b, h): the homogeneity identity sum<x, dx> = sum<do, o> (o is degree 1 in each of q, k, v),
    as two ratios.  gated: |sum<x, dx> - sum<do, o>| / ||x * dx||_2, the difference against the
    natural size of a sum of that many terms of either sign (a gradient of the right size but
    wrong signs or places still gives a ratio near 1).  cond: the same difference over
    |sum<do, o>|, reported only: that sum cancels, so where it happens to be small the ratio grows
    with no error in dx."""
    prod = x.double() * dx.double()
    diff = (prod.sum(dim=(2, 3)) - ref).abs()
    scale = prod.pow(2).sum(dim=(2, 3)).sqrt()
    del prod
    return (diff / scale)[0].tolist(), (diff / ref.abs())[0].tolist()


def check(gpu, ref, keys, tol, label):
    errs = {n: maxrel(gpu[n], ref[n]) for n in keys}
    say(label, " ".join("%s=%.2e(el %.1e)" % (n, e, elemrel(gpu[n], ref[n])) for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, "%s: max relative error above %.0e: %s" % (label, tol, bad)


def run_case(B, H, T, dk, dv, chunk, P, K, dtype, bwd, gate="logsigmoid16", seed=0, carry=False):
    d = inputs.generate(B, H, T, dk, dv, dtype, seed, bwd, gate)
    h0 = dhT = None
    if carry:
        rng = np.random.default_rng(seed + 100)
        h0 = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3)
        dhT = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3)
    gpu = gpu_pipeline(dev(d), chunk, P, K, bwd, None if h0 is None else h0.cuda(),
                       None if dhT is None else dhT.cuda())
    ref = oracle_pipeline(d, chunk, P, bwd, None if h0 is None else h0.numpy(), None if dhT is None else dhT.numpy())
    label = "B%d H%d T%d dk%d dv%d C%d P%d K%d %s %s" % (B, H, T, dk, dv, chunk, P, K, dtype, gate)
    check(gpu, ref, FWD_KEYS + (BWD_KEYS if bwd else ()), TOL[dtype], label)
    # and the end result against the plain recurrence, without any segmentation
    a = {n: as_f64(t) for n, t in d.items()}
    o, hT = oracle.gla_fwd(a["q"], a["k"], a["v"], a["g"], None if h0 is None else h0.numpy())
    plain = {"o": o, "h_final": hT}
    keys = ("o", "h_final")
    if bwd:
        plain.update(oracle.gla_bwd(a["q"], a["k"], a["v"], a["g"], a["do"], None if h0 is None else h0.numpy(),
                                    None if dhT is None else dhT.numpy()))
        keys += ("dq", "dk", "dv", "dg", "dh0")
    check(gpu, plain, keys, TOL[dtype], label + " vs plain recurrence")
    return gpu


# ------------------------------------------------------------------------------- the workloads

def test_tiny_fp32_workload():
    w = inputs.WORKLOADS["tiny_fp32_t256_p4"]
    run_case(w.B, w.H, w.T, w.dk, w.dv, w.chunk, w.P, w.K, w.dtype, bwd=False)
    # the same shape through the backward as well
    run_case(w.B, w.H, w.T, w.dk, w.dv, w.chunk, w.P, w.K, w.dtype, bwd=True)


@pytest.mark.parametrize("name", ["fwd_b2h4_t16k_p1", "fwd_h4_t32k_p8"])
def test_forward_workloads(name):
    w = inputs.WORKLOADS[name]
    t = time.time()
    run_case(w.B, w.H, w.T, w.dk, w.dv, w.chunk, w.P, w.K, w.dtype, bwd=False)
    say("%s: %.1fs" % (name, time.time() - t))


def test_fwdbwd_workload_h16():
    w = inputs.WORKLOADS["fwdbwd_h16_t16k_p4"]
    t = time.time()
    gpu = run_case(w.B, w.H, w.T, w.dk, w.dv, w.chunk, w.P, w.K, w.dtype, bwd=True)
    say("%s: %.1fs" % (w.name, time.time() - t))


@pytest.mark.parametrize("name", ["tiny_fp32_t256_p4", "fwd_b2h4_t16k_p1", "fwd_h4_t32k_p8", "fwdbwd_h16_t16k_p4"])
def test_workloads_in_the_states_first_order(name):
    """The smaller workloads at full size through the states-first chain the benchmark times
    (gla.states_first_forward / _backward, segments cut to fill the chip), against the oracle's
    plain recurrence over every token: o and h_final, and with the backward dq, dk, dv, dg and dh0
    (the backward runs on every workload, the forward-only ones included)."""
    w = inputs.WORKLOADS[name]
    d = inputs.generate_workload(w, bwd=True)
    x = dev(d)
    t = time.time()
    f = gla.states_first_forward(x["q"], x["k"], x["v"], x["g"], w.chunk, w.P, w.K)
    b = gla.states_first_backward(x["q"], x["k"], x["v"], x["g"], x["do"], f, w.chunk, w.K)
    torch.cuda.synchronize()
    say("%s states first: P' = %d, %.1fs" % (name, f["P"], time.time() - t))
    gpu = {"o": as_f64(f["o"]), "h_final": as_f64(f["h_final"])}
    gpu.update({n: as_f64(b[n]) for n in ("dq", "dk", "dv", "dg", "dh0")})
    a = {n: as_f64(v) for n, v in d.items()}
    o, hT = oracle.gla_fwd(a["q"], a["k"], a["v"], a["g"])
    ref = {"o": o, "h_final": hT}
    ref.update(oracle.gla_bwd(a["q"], a["k"], a["v"], a["g"], a["do"]))
    check(gpu, ref, ("o", "h_final", "dq", "dk", "dv", "dg", "dh0"), TOL[w.dtype], "%s, states first" % name)


# ------------------------------------------------------------------------- stress and edge cases

@pytest.mark.parametrize("gate", ["weak", "zero", "strong", "strong5", "mixed", "scalar"])
@pytest.mark.parametrize("dtype,dk,dv,chunk", [("bf16", 64, 128, 32), ("bf16", 64, 128, 64), ("bf16", 64, 128, 16),
                                                ("f32", 32, 16, 16), ("f32", 32, 16, 32), ("f32", 32, 16, 64)])
def test_gate_variants_with_boundary_states(gate, dtype, dk, dv, chunk):
    # B*H = 3 units per segment (not a multiple of the 8-way XCD grouping), h0 and dL/dS_T given.
    # strong (about -2 per token) and strong5 (about -5 per token, the survey's stress gate) decay
    # far beyond what the chunk factorisation takes: those units run the exact sub-block kernels
    run_case(1, 3, 1024, dk, dv, chunk, 4, 2, dtype, bwd=True, gate=gate, seed=5, carry=True)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_strong_decay_at_the_headline_head_shape(chunk):
    # g = min(-5 + x/4, 0) at d_k = 128, d_v = 256: the whole path, with boundary states, against the
    # oracle (every chunk decays by e^-80 per 16 tokens or more)
    run_case(1, 2, 2048, 128, 256, chunk, 4, 2, "bf16", bwd=True, gate="strong5", seed=13, carry=True)


def test_fast_and_exact_units_in_one_call():
    # a strong window inside some segments only: in one call the fast kernels take the other units
    # and the exact kernels these (their flags set mid-segment, forward and backward)
    B, H, T, dk, dv, chunk, P = 1, 3, 2048, 64, 128, 64, 4
    d = inputs.generate(B, H, T, dk, dv, "bf16", 17, True, "weak")
    g = d["g"].clone()
    g[0, 0, 300:340] = -3.0       # segment 0 of head 0, inside one chunk and across a chunk edge
    g[0, 2, 1500:1530, ::3] = -4.0  # segment 2 of head 2, some channels only
    d["g"] = g
    x = dev(d)
    gpu = gpu_pipeline(x, chunk, P, 2, True)
    ref = oracle_pipeline(d, chunk, P, True)
    check(gpu, ref, FWD_KEYS + BWD_KEYS, TOL["bf16"], "fast and exact units in one call")


@pytest.mark.parametrize("dtype,dk,dv,chunk,P", [("bf16", 32, 32, 32, 8), ("bf16", 128, 256, 64, 3),
                                                  ("f32", 16, 32, 32, 5), ("f32", 32, 32, 64, 1)])
def test_one_chunk_per_segment_and_odd_counts(dtype, dk, dv, chunk, P):
    run_case(2, 1, chunk * P, dk, dv, chunk, P, 1, dtype, bwd=True, gate="weak", seed=6)


SUPPORTED = ([("bf16", dk, dv, c) for dk in (32, 64, 128) for dv in (32, 64, 128, 256) for c in (16, 32, 64)] +
             [("f32", dk, dv, c) for dk in (16, 32) for dv in (16, 32) for c in (16, 32, 64)])


@pytest.mark.parametrize("dtype,dk,dv,chunk", SUPPORTED)
def test_every_supported_shape(dtype, dk, dv, chunk):
    # every compiled kernel instantiation, fwd+bwd through all steps, against the oracle: 4
    # segments of 2 chunks, boundary states given
    assert gla.load_library().gla_supported(gla.GLA_BF16 if dtype == "bf16" else gla.GLA_F32, dk, dv, chunk) == 1
    run_case(1, 2, 8 * chunk, dk, dv, chunk, 4, 2, dtype, bwd=True, gate="weak", seed=21, carry=True)


def _mixed_cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        dtype, dk, dv, chunk = SUPPORTED[int(rng.integers(len(SUPPORTED)))]
        B, H, P = int(rng.integers(1, 4)), int(rng.integers(1, 6)), int(rng.integers(1, 10))
        per_seg = int(rng.integers(1, 6))
        K = [k for k in (1, 2, 4, 8, 16) if dk % k == 0][int(rng.integers(0, 3))]
        gate = ("logsigmoid16", "weak", "strong", "scalar", "strong5")[int(rng.integers(5))]
        cases.append((B, H, P * per_seg * chunk, dk, dv, chunk, P, K, dtype, gate, int(rng.integers(1000))))
    return cases


@pytest.mark.parametrize("case", _mixed_cases())
def test_mixed_configurations(case):
    # a fixed sample of mixed shapes, segment counts, batch/head counts, dtypes and gates, fwd+bwd
    # with boundary states, against the oracle step by step and against the plain recurrence
    B, H, T, dk, dv, chunk, P, K, dtype, gate, seed = case
    run_case(B, H, T, dk, dv, chunk, P, K, dtype, bwd=True, gate=gate, seed=seed, carry=True)


def test_chunk_size_invariance():
    d = dev(inputs.generate(1, 2, 2048, 128, 128, "bf16", 3, True, "weak"))
    a = gpu_pipeline(d, 32, 4, 4, True)
    b = gpu_pipeline(d, 64, 4, 4, True)
    for n in ("o", "dq", "dk", "dv", "dg", "h_final"):
        assert maxrel(a[n], b[n]) <= TOL["bf16"], n


def test_run_to_run_determinism():
    d = dev(inputs.generate(1, 4, 4096, 128, 256, "bf16", 4, True))
    a = gpu_pipeline(d, 64, 4, 2, True)
    b = gpu_pipeline(d, 64, 4, 2, True)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("gate", ["logsigmoid16", "strong", "zero"])
def test_corrections_are_bitwise_independent_of_the_split(gate):
    """Where B*H*P leaves CUs idle, both corrections cut each segment into sub-segments.  64 heads x
    4 segments (256 units) run uncut; 16- and 4-head slices of the same tensors run cut into 4 and 16
    sub-segments (16 and 1 chunks each).  The results must agree bit for bit, whether the decay dies inside the segment
    (strong) or never (zero)."""
    B, H, T, dk, dv, chunk, P = 1, 64, 4096, 128, 256, 64, 4
    d = dev(inputs.generate(B, H, T, dk, dv, "bf16", 21, True, gate))
    q, k, v, g = d["q"], d["k"], d["v"], d["g"]
    rng = np.random.default_rng(5)
    h0 = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3).cuda()
    dhT = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3).cuda()
    o, cs, S_loc, ld = gla.gla_chunk_fwd(q, k, v, g, chunk, P)
    S_in, _ = gla.gla_segment_scan(S_loc, ld, 1, h_boundary=h0)
    o_loc, cs_loc = o.clone(), cs.clone()
    gla.gla_segment_correct(gla.GLA_FWD, chunk, P, q=q, g=g, seg_in=S_in, o=o, chunk_states=cs)
    dq, dk_, dv_, dg, D = gla.gla_chunk_bwd(q, k, v, g, d["do"], cs, S_in, chunk, P)
    G, _ = gla.gla_segment_scan(D, ld, 1, h_boundary=dhT, reverse=True)
    local = (dk_.clone(), dv_.clone(), dg.clone())
    gla.gla_segment_correct(gla.GLA_BWD, chunk, P, k=k, v=v, g=g, seg_in=S_in, seg_grad=G, chunk_states=cs,
                            dk=dk_, dv=dv_, dg=dg)
    for nh in (16, 4):
        for h in (0, H - nh):
            sl = slice(h, h + nh)

            def part(t):  # a copy: with B = 1 a head slice is already contiguous, and the calls write in place
                return t[:, sl].clone(memory_format=torch.contiguous_format)

            o2, cs2 = part(o_loc), part(cs_loc)
            gla.gla_segment_correct(gla.GLA_FWD, chunk, P, q=part(q), g=part(g), seg_in=part(S_in), o=o2,
                                    chunk_states=cs2)
            dk2, dv2, dg2 = (part(t) for t in local)
            gla.gla_segment_correct(gla.GLA_BWD, chunk, P, k=part(k), v=part(v), g=part(g), seg_in=part(S_in),
                                    seg_grad=part(G), chunk_states=part(cs), dk=dk2, dv=dv2, dg=dg2)
            torch.cuda.synchronize()
            say("heads %d..%d of %d %s: o %s cs %s dk %s dv %s dg %s" % (
                h, h + nh - 1, H, gate, *(bool(torch.equal(x, y[:, sl])) for x, y in
                                          ((o2, o), (cs2, cs), (dk2, dk_), (dv2, dv_), (dg2, dg)))))
            for x, y, n in ((o2, o, "o"), (cs2, cs, "chunk_states"), (dk2, dk_, "dk"), (dv2, dv_, "dv"),
                            (dg2, dg, "dg")):
                assert torch.equal(x, y[:, sl]), "%s differs with the split (heads %d..%d)" % (n, h, h + nh - 1)


@pytest.mark.parametrize("B,H,T,dk,dv,chunk,P,dtype,gate", [
    (1, 4, 1 << 16, 128, 256, 64, 64, "bf16", "logsigmoid16"),  # 256 units: uncut
    (2, 4, 16384, 128, 256, 64, 1, "bf16", "logsigmoid16"),     # cut into sub-segments
    (1, 3, 1024, 64, 128, 32, 4, "bf16", "strong5"),            # the exact kernels
    (1, 3, 1024, 64, 128, 16, 4, "bf16", "weak"),               # bf16 chunk 16: exact kernels
    (1, 3, 1024, 32, 16, 32, 4, "f32", "logsigmoid16")])
def test_forward_without_chunk_states(B, H, T, dk, dv, chunk, P, dtype, gate):
    """A forward-only caller keeps no per-chunk states (chunk_states NULL through the C ABI): the
    local outputs, segment states and log-decays, and the corrected outputs, equal the run that
    keeps them bit for bit; and the backward refuses to run without them."""
    d = dev(inputs.generate(B, H, T, dk, dv, dtype, 3, False, gate))
    q, k, v, g = d["q"], d["k"], d["v"], d["g"]
    rng = np.random.default_rng(8)
    h0 = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3).cuda()
    with_cs = gla.zeco_forward(q, k, v, g, chunk, P, 1, h0=h0)
    no_cs = gla.zeco_forward(q, k, v, g, chunk, P, 1, h0=h0, keep_chunk_states=False)
    loc = gla.gla_chunk_fwd(q, k, v, g, chunk, P, keep_chunk_states=False)
    loc_cs = gla.gla_chunk_fwd(q, k, v, g, chunk, P)
    torch.cuda.synchronize()
    assert no_cs["chunk_states"] is None and loc[1] is None
    for n in ("o", "seg_state", "seg_logdecay", "seg_in", "h_final"):
        assert torch.equal(no_cs[n], with_cs[n]), n
    for i, n in ((0, "o_local"), (2, "seg_state"), (3, "seg_logdecay")):
        assert torch.equal(loc[i], loc_cs[i]), n
    with pytest.raises(ValueError):
        gla.gla_chunk_bwd(q, k, v, g, torch.zeros_like(v), None, no_cs["seg_in"], chunk, P)
    with pytest.raises(ValueError):
        gla.gla_chunk_fwd(q, k, v, g, chunk, P, chunk_states=loc_cs[1], keep_chunk_states=False)


def test_scan_is_bitwise_independent_of_K():
    rng = np.random.default_rng(9)
    B, H, P, dk, dv = 2, 3, 7, 64, 48
    S = torch.from_numpy(rng.standard_normal((B, H, P, dk, dv)).astype(np.float32)).cuda()
    ld = torch.from_numpy((-np.abs(rng.standard_normal((B, H, P, dk))) * 0.5).astype(np.float32)).cuda()
    h = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32)).cuda()
    for rev in (False, True):
        outs = [gla.gla_segment_scan(S, ld, K, h_boundary=h, reverse=rev) for K in (1, 2, 4, 8, 16, 64)]
        torch.cuda.synchronize()
        for c, o in outs[1:]:
            assert torch.equal(c, outs[0][0]) and torch.equal(o, outs[0][1])
        ref_c, ref_h = oracle.segment_scan(as_f64(S), as_f64(ld), as_f64(h), reverse=rev)
        assert maxrel(as_f64(outs[0][0]), ref_c) < 1e-5
        assert maxrel(as_f64(outs[0][1]), ref_h) < 1e-5


@pytest.mark.parametrize("P", [1, 2, 7, 64])
def test_allgather_scan_matches_oracle_and_chain(P):
    # the all-gather ordering of the scan: the oracle's chain to float32 rounding, for both
    # directions, with and without boundary states
    rng = np.random.default_rng(11 + P)
    B, H, dk, dv = 2, 3, 32, 48
    S = torch.from_numpy(rng.standard_normal((B, H, P, dk, dv)).astype(np.float32)).cuda()
    ld = torch.from_numpy((-np.abs(rng.standard_normal((B, H, P, dk))) * 0.3).astype(np.float32)).cuda()
    h = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32)).cuda()
    for rev in (False, True):
        for hb in (None, h):
            c_ag, h_ag = gla.gla_segment_scan_allgather(S, ld, h_boundary=hb, reverse=rev)
            c_ch, h_ch = gla.gla_segment_scan(S, ld, 4, h_boundary=hb, reverse=rev)
            torch.cuda.synchronize()
            ref_c, ref_h = oracle.segment_scan(as_f64(S), as_f64(ld), None if hb is None else as_f64(hb), reverse=rev)
            for got, ref in ((c_ag, ref_c), (h_ag, ref_h), (c_ag, as_f64(c_ch)), (h_ag, as_f64(h_ch))):
                assert maxrel(as_f64(got), ref) < 1e-5, (P, rev, hb is None)


def test_allgather_pipeline_matches_chain_pipeline():
    d = dev(inputs.generate(1, 2, 4096, 64, 128, "bf16", 12, True))
    fc = gla.zeco_forward(d["q"], d["k"], d["v"], d["g"], 64, 8, 4)
    bc = gla.zeco_backward(d["q"], d["k"], d["v"], d["g"], d["do"], fc, 64, 8, 4)
    fa = gla.zeco_forward(d["q"], d["k"], d["v"], d["g"], 64, 8, 4, scan="allgather")
    ba = gla.zeco_backward(d["q"], d["k"], d["v"], d["g"], d["do"], fa, 64, 8, 4, scan="allgather")
    torch.cuda.synchronize()
    for n in ("o", "h_final"):
        assert maxrel(as_f64(fa[n]), as_f64(fc[n])) <= TOL["bf16"], n
    for n in ("dq", "dk", "dv", "dg", "dh0"):
        assert maxrel(as_f64(ba[n]), as_f64(bc[n])) <= TOL["bf16"], n


@pytest.mark.parametrize("n_streams", [2, 3])
def test_multi_stream_schedule(n_streams):
    # the sequences split over several streams, each group's six calls on its own stream: bit for
    # bit the one-stream chain with flag-only workspaces (no sub-segments, as the groups run), and
    # the oracle's results (boundary states given, one group of sequences taking the exact kernels
    # through a strongly decaying stretch)
    B, H, T, dk, dv, chunk, P, K = 2, 3, 2048, 64, 128, 64, 4, 2
    d = inputs.generate(B, H, T, dk, dv, "bf16", 19, True, "logsigmoid16")
    d["g"][1, 2, 700:760] = -3.0
    rng = np.random.default_rng(3)
    h0 = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3)
    dhT = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3)
    x = dev(d)
    got = gla.zeco_step_streams(x["q"], x["k"], x["v"], x["g"], x["do"], chunk, P, K, n_streams,
                                h0=h0.cuda(), dhT=dhT.cuda())
    ws = torch.empty(gla.flags_workspace_size(B, H, P), dtype=torch.uint8, device="cuda")
    one = gpu_pipeline(x, chunk, P, K, True, h0.cuda(), dhT.cuda(), ws=ws)
    torch.cuda.synchronize()
    names = {"o": "o", "h_final": "h_final", "dq": "dq", "dk": "dk", "dv": "dv", "dg": "dg", "dh0": "dh0",
             "seg_in": "S_in", "seg_grad": "G"}
    for a_, b_ in names.items():
        assert np.array_equal(as_f64(got[a_]), one[b_]), a_
    ref = oracle_pipeline(d, chunk, P, True, h0.numpy(), dhT.numpy())
    check({k_: one[k_] for k_ in ("o", "h_final", "dq", "dk", "dv", "dg", "dh0")}, ref,
          ("o", "h_final", "dq", "dk", "dv", "dg", "dh0"), TOL["bf16"], "%d streams" % n_streams)


def _layout(units, dk, dv, S, R=0):
    """The workspace rule of include/gla.h (gla_workspace_size) for S sub-segments per segment and R
    re-split slots: the byte offset of the re-split's list, and the total."""
    a = lambda n: (n + 255) // 256 * 256  # noqa: E731
    u = units * S
    off = a(4 * u) + (a(4 * u * dk * dv) + a(4 * u * dk) + a(4 * u * dk * dv) if S > 1 else 0)
    total = off + (a(4 * (2 + R)) + a(4 * R * dk * dv) + a(4 * R * dk) + a(4 * R * dk * dv) if R else 0)
    return off, total


def _layout_bytes(units, dk, dv, S):
    return _layout(units, dk, dv, S)[1]


def test_small_workspace_runs_fewer_sub_segments():
    """A workspace below gla_workspace_size (down to the flags) runs fewer sub-segments, or none.
    8 units of 32 chunks are cut into 16 with the full workspace; here also into 4 and 1.  Every
    run matches the oracle, the runs agree to rounding, and the flags-only forward equals
    gla_chunk_fwd_noalloc (which never cuts) bit for bit."""
    B, H, T, dk, dv, chunk, P, K = 2, 2, 4096, 64, 128, 64, 2, 1
    d = inputs.generate(B, H, T, dk, dv, "bf16", 23, True, "logsigmoid16")
    x = dev(d)
    full = gla.workspace_size(gla.GLA_BWD, B, H, T, dk, dv, chunk, P, torch.bfloat16)
    assert full == _layout_bytes(B * H * P, dk, dv, 16)
    ref = oracle_pipeline(d, chunk, P, True)
    runs = {}
    for S in (16, 4, 1):
        ws = torch.empty(_layout_bytes(B * H * P, dk, dv, S) + (255 if S < 16 else 0), dtype=torch.uint8,
                         device="cuda")
        runs[S] = gpu_pipeline(x, chunk, P, K, True, ws=ws)
        check(runs[S], ref, FWD_KEYS + BWD_KEYS, TOL["bf16"], "workspace for %d sub-segments" % S)
    for S in (4, 1):
        for n in ("o", "dq", "dk", "dv", "dg"):
            assert maxrel(runs[S][n], runs[16][n]) < 1e-2, (S, n)  # bf16 outputs: a few ulps
    o = torch.empty_like(x["v"])
    cs = torch.empty((B, H, T // chunk, dk, dv), dtype=torch.bfloat16, device="cuda")
    st = torch.empty((B, H, P, dk, dv), device="cuda")
    ld = torch.empty((B, H, P, dk), device="cuda")
    gla.gla_chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["g"], chunk, P, o, cs, st, ld)
    torch.cuda.synchronize()
    assert np.array_equal(as_f64(o), runs[1]["o_local"]) and np.array_equal(as_f64(st), runs[1]["S_local"])
    with pytest.raises(gla.GLAError):  # below the flags
        gla.gla_chunk_fwd(x["q"], x["k"], x["v"], x["g"], chunk, P,
                          workspace=torch.empty(255, dtype=torch.uint8, device="cuda"))


# (dtype, B, H, T, dk, dv, chunk, P, gate, strong units, S, R, n, X): strong units are the units
# (b, h, segment, sub-segment) that get a strongly decaying stretch (None: the gate decays strongly
# everywhere); S the sub-segments per segment, R the re-split slots; n units listed, X pieces each.
RESPLIT_CASES = [
    # 256 units of 16 chunks: two flagged, 8 pieces each
    ("bf16", 1, 4, 65536, 64, 64, 64, 64, "logsigmoid16", [3, 200], 1, 256, 2, 8),
    # forty flagged: 4 pieces each
    ("bf16", 1, 4, 65536, 32, 32, 64, 64, "logsigmoid16", list(range(0, 240, 6)), 1, 256, 40, 4),
    # 512 units, all flagged: the first 256 listed whole, the rest in the plain exact pass
    ("bf16", 2, 4, 32768, 32, 32, 64, 64, "strong5", None, 1, 256, 256, 1),
    # 8 segments cut into 32 sub-segments of 8 chunks; one sub-segment flagged, 4 pieces
    ("bf16", 1, 2, 65536, 64, 64, 64, 4, "logsigmoid16", [77], 32, 256, 1, 4),
    # every sub-segment flagged: listed whole, each from the sub-segment split's incoming state
    ("bf16", 1, 2, 65536, 64, 64, 64, 4, "strong5", None, 32, 256, 256, 1),
    ("f32", 1, 4, 32768, 32, 32, 32, 64, "logsigmoid16", [5, 130, 131], 1, 256, 3, 8),
]


@pytest.mark.parametrize("case", RESPLIT_CASES, ids=lambda c: "%s-T%d-P%d-%s-n%d" % (c[0], c[3], c[7], c[8], c[12]))
def test_flagged_units_are_re_split(case):
    """Units the fast kernels flag are cut into pieces and redone from each piece's true incoming
    state: the whole path matches the oracle, the workspace's list names the flagged units and the
    piece count the rule gives, and a flags-only workspace (no re-split) agrees to rounding."""
    dtype, B, H, T, dk, dv, chunk, P, gate, strong, S, R, n, X = case
    d = inputs.generate(B, H, T, dk, dv, dtype, 29, True, gate)
    units = B * H * P * S
    Ls = T // P // S
    if strong is not None:
        g = d["g"].clone()
        for u in strong:  # a stretch of 48 tokens decaying by e^-3 per token in every other channel
            b, rest = divmod(u, H * P * S)
            h, rest = divmod(rest, P * S)
            t0 = rest * Ls + Ls // 2 - 24
            g[b, h, t0:t0 + 48, ::2] = -3.0
        d["g"] = g
    x = dev(d)
    full = gla.workspace_size(gla.GLA_BWD, B, H, T, dk, dv, chunk, P, x["q"].dtype)
    list_at, total = _layout(B * H * P, dk, dv, S, R)
    assert full == total
    ws = torch.empty(full, dtype=torch.uint8, device="cuda")
    say("re-split case", case[:9], "units", units)
    gpu = gpu_pipeline(x, chunk, P, 2, True, ws=ws)
    lst = ws[list_at:list_at + 4 * (2 + n)].view(torch.int32).cpu().numpy()  # the backward's list
    expect = list(range(n)) if strong is None else sorted(strong)
    assert lst[0] == n and lst[1] == X and list(lst[2:]) == expect, (lst[:2], lst[2:12])
    ref = oracle_pipeline(d, chunk, P, True)
    check(gpu, ref, FWD_KEYS + BWD_KEYS, TOL[dtype], "re-split %s" % (case[:9],))
    flags_only = torch.empty(gla.flags_workspace_size(B, H, P) if S == 1 else _layout_bytes(B * H * P, dk, dv, S),
                             dtype=torch.uint8, device="cuda")
    plain = gpu_pipeline(x, chunk, P, 2, True, ws=flags_only)
    for k_ in ("o", "dq", "dk", "dv", "dg", "S_local", "D_local"):
        assert maxrel(gpu[k_], plain[k_]) < TOL[dtype] / 2, k_


# -------------------------------------------------------- the order with the incoming states first

SF_FWD_KEYS = ("S_local", "logdecay", "S_in", "h_final", "o", "cs")
SF_BWD_KEYS = ("D_local", "G", "dh0", "dq", "dk", "dv", "dg")
REACH_CUT = -112.0  # below it exp gives 0.0f: the state passes stop once every channel is past it


def reach_clamped(res):
    """The states-first state pass stops once every channel's summed log-gates are below the cut
    and then reports the sum over the chunks it walked; past the cut only the (zero) exponential
    is defined, so log-decays are compared clamped at the cut."""
    out = dict(res)
    out["logdecay"] = np.maximum(res["logdecay"], REACH_CUT)
    return out


def states_first_pipeline(d, chunk, P, K, h0=None, dhT=None, ws=None):
    """State pass -> scan -> local pass from each segment's true incoming state, and the same for
    the backward, through the C ABI, keeping the intermediates (float64 numpy arrays)."""
    q, k, v, g = d["q"], d["k"], d["v"], d["g"]
    S_loc, ld = gla.gla_chunk_state(k, v, g, chunk, P, workspace=ws)
    S_in, h_final = gla.gla_segment_scan(S_loc, ld, K, h_boundary=h0)
    o, cs = gla.gla_chunk_fwd_from(q, k, v, g, S_in, chunk, P, workspace=ws)
    res = {"S_local": S_loc, "logdecay": ld, "S_in": S_in, "h_final": h_final, "o": o,
           "cs": gla.chunk_states_dense(cs)}
    D = gla.gla_chunk_dstate(q, g, d["do"], chunk, P, workspace=ws)
    G, dh0 = gla.gla_segment_scan(D, ld, K, h_boundary=dhT, reverse=True)
    dq, dk, dv, dg = gla.gla_chunk_bwd_from(q, k, v, g, d["do"], cs, S_in, G, chunk, P, workspace=ws)
    res.update(D_local=D, G=G, dh0=dh0, dq=dq, dk=dk, dv=dv, dg=dg)
    torch.cuda.synchronize()
    return {n: as_f64(t) for n, t in res.items()}


SF_CASES = [
    # dtype, B, H, T, dk, dv, chunk, P, K, gate
    ("bf16", 1, 4, 16384, 64, 64, 64, 64, 8, "logsigmoid16"),   # 256 units, no sub-segments
    ("bf16", 1, 2, 4096, 128, 256, 64, 4, 2, "logsigmoid16"),   # 8 units, each cut into 8 sub-segments
    ("bf16", 2, 1, 8192, 64, 128, 32, 4, 4, "zero"),
    ("bf16", 1, 2, 4096, 64, 128, 64, 4, 2, "strong5"),         # every unit on the exact kernels
    ("bf16", 1, 2, 4096, 64, 128, 64, 4, 2, "mixed"),
    ("bf16", 1, 2, 2048, 64, 128, 16, 4, 2, "logsigmoid16"),    # chunk 16: the state passes run in 64-token chunks
    ("bf16", 1, 1, 960, 32, 32, 64, 3, 1, "weak"),              # 5 chunks a segment: no sub-segments
    ("f32", 1, 2, 1024, 32, 32, 16, 4, 2, "strong"),
    ("f32", 1, 1, 256, 16, 16, 16, 4, 2, "logsigmoid16"),       # the tiny configuration
]


@pytest.mark.parametrize("case", SF_CASES, ids=lambda c: "%s-T%d-dk%d-dv%d-C%d-P%d-%s" % (c[0], c[3], c[4], c[5],
                                                                                          c[6], c[7], c[9]))
def test_states_first_order_matches_oracle(case):
    """gla_chunk_state -> gla_segment_scan -> gla_chunk_fwd_from and gla_chunk_dstate -> reverse scan
    -> gla_chunk_bwd_from, with boundary states h0 and dL/dS_T: every intermediate and result
    against the oracle's segmented form, and against the correction order on the same inputs."""
    dtype, B, H, T, dk, dv, chunk, P, K, gate = case
    d = inputs.generate(B, H, T, dk, dv, dtype, 41, True, gate)
    rng = np.random.default_rng(141)
    h0 = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3)
    dhT = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3)
    x = dev(d)
    gpu = states_first_pipeline(x, chunk, P, K, h0.cuda(), dhT.cuda())
    ref = oracle_pipeline(d, chunk, P, True, h0.numpy(), dhT.numpy())
    label = "states first %s B%d H%d T%d dk%d dv%d C%d P%d %s" % (dtype, B, H, T, dk, dv, chunk, P, gate)
    check(reach_clamped(gpu), reach_clamped(ref), SF_FWD_KEYS + SF_BWD_KEYS, TOL[dtype], label)
    zc = gpu_pipeline(x, chunk, P, K, True, h0.cuda(), dhT.cuda())
    check(reach_clamped(gpu), reach_clamped(zc), SF_FWD_KEYS + SF_BWD_KEYS, TOL[dtype],
          label + " vs the correction order")


@pytest.mark.parametrize("gate", ["logsigmoid16", "mixed", "strong5", "weak"])
def test_state_passes_stop_where_the_decay_ends(gate):
    """Segments of 128 chunks with only the flags as workspace (no sub-segments): the state passes
    walk from the far end and stop once every channel is past the cut.  The states and gradients
    must still match the oracle; where the oracle's log-decay is far below the cut the reported
    one is the partial sum, between the cut and the full sum (so the walk did stop early); where
    the walk reached the segment's start it is the full sum."""
    B, H, T, dk, dv, chunk, P = 1, 2, 16384, 64, 128, 64, 2
    d = inputs.generate(B, H, T, dk, dv, "bf16", 47, True, gate)
    rng = np.random.default_rng(147)
    h0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3
    dhT = rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3
    x = dev(d)
    ws = torch.zeros(gla.flags_workspace_size(B, H, P), dtype=torch.uint8, device="cuda")
    gpu = states_first_pipeline(x, chunk, P, 2, torch.from_numpy(h0).cuda(), torch.from_numpy(dhT).cuda(), ws=ws)
    ref = oracle_pipeline(d, chunk, P, True, h0, dhT)
    check(reach_clamped(gpu), reach_clamped(ref), SF_FWD_KEYS + SF_BWD_KEYS, TOL["bf16"], "reach %s" % gate)
    ld, ld_ref = gpu["logdecay"], ref["logdecay"]
    full = (ld >= REACH_CUT).any(axis=-1)  # segments whose walk reached the start: every sum complete
    assert np.allclose(ld[full], ld_ref[full], rtol=1e-5, atol=1e-3)
    if gate in ("logsigmoid16", "strong5"):  # every channel decays past the cut (mixed: only half)
        far = ld_ref < 2 * REACH_CUT
        assert far.all(axis=-1).any(), "this gate should decay past the cut within a segment"
        assert (ld[~full] < REACH_CUT).all() and (ld[~full] >= ld_ref[~full] - 1e-3).all()
        assert (ld[far & ~full[..., None]] > ld_ref[far & ~full[..., None]] + 1.0).any(), "the walk never stopped"


def test_states_first_order_re_splits_flagged_units():
    """Strong stretches in two of 256 units: the fast kernels flag them and the re-split redoes
    them in pieces, each from its true incoming state, the segment's first piece from seg_in."""
    B, H, T, dk, dv, chunk, P = 1, 4, 65536, 64, 64, 64, 64
    d = inputs.generate(B, H, T, dk, dv, "bf16", 29, True, "logsigmoid16")
    g = d["g"].clone()
    L = T // P
    for u in (3, 200):
        h, p = divmod(u, P)
        t0 = p * L + L // 2 - 24
        g[0, h, t0:t0 + 48, ::2] = -3.0
    d["g"] = g
    x = dev(d)
    full = gla.workspace_size(gla.GLA_BWD, B, H, T, dk, dv, chunk, P, x["q"].dtype)
    list_at, total = _layout(B * H * P, dk, dv, 1, 256)
    assert full == total
    ws = torch.empty(full, dtype=torch.uint8, device="cuda")
    gpu = states_first_pipeline(x, chunk, P, 2, ws=ws)
    lst = ws[list_at:list_at + 16].view(torch.int32).cpu().numpy()  # the backward's list
    assert lst[0] == 2 and lst[1] == 8 and list(lst[2:]) == [3, 200], lst
    ref = oracle_pipeline(d, chunk, P, True)
    check(reach_clamped(gpu), reach_clamped(ref), SF_FWD_KEYS + SF_BWD_KEYS, TOL["bf16"], "states first, re-split")


def test_states_first_chain_fills_the_chip():
    """gla.states_first_forward / states_first_backward cut the 8 units (2 segments of 4 heads) into
    256 segments of 2 chunks, so that no call cuts sub-segments of its own: the results against the
    plain recurrence, with boundary states."""
    B, H, T, dk, dv, chunk, P = 1, 4, 32768, 64, 128, 64, 2
    d = inputs.generate(B, H, T, dk, dv, "bf16", 43, True, "logsigmoid16")
    rng = np.random.default_rng(143)
    h0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3
    dhT = rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3
    x = dev(d)
    f = gla.states_first_forward(x["q"], x["k"], x["v"], x["g"], chunk, P, 4, h0=torch.from_numpy(h0).cuda())
    assert f["P"] == 64 and f["seg_state"].shape[2] == 64
    b = gla.states_first_backward(x["q"], x["k"], x["v"], x["g"], x["do"], f, chunk, 4,
                                  dhT=torch.from_numpy(dhT).cuda())
    torch.cuda.synchronize()
    gpu = {"o": as_f64(f["o"]), "h_final": as_f64(f["h_final"])}
    gpu.update({n: as_f64(b[n]) for n in ("dq", "dk", "dv", "dg", "dh0")})
    a = {n: as_f64(t) for n, t in d.items()}
    o, hT = oracle.gla_fwd(a["q"], a["k"], a["v"], a["g"], h0)
    ref = {"o": o, "h_final": hT}
    ref.update(oracle.gla_bwd(a["q"], a["k"], a["v"], a["g"], a["do"], h0, dhT))
    check(gpu, ref, ("o", "h_final", "dq", "dk", "dv", "dg", "dh0"), TOL["bf16"], "states-first chain, P' = 64")


def test_state_carry_across_calls():
    # running the second half with h0 = the first half's final state equals one call
    d = inputs.generate(1, 2, 2048, 64, 64, "bf16", 8, False, "weak")
    full = gla.zeco_forward(*(d[n].cuda() for n in ("q", "k", "v", "g")), 64, 2, 2)
    first = gla.zeco_forward(*(d[n][:, :, :1024].contiguous().cuda() for n in ("q", "k", "v", "g")), 64, 1, 1)
    second = gla.zeco_forward(*(d[n][:, :, 1024:].contiguous().cuda() for n in ("q", "k", "v", "g")), 64, 1, 1,
                              h0=first["h_final"])
    torch.cuda.synchronize()
    o = torch.cat([first["o"], second["o"]], dim=2)
    assert maxrel(as_f64(o), as_f64(full["o"])) <= TOL["bf16"]
    assert maxrel(as_f64(second["h_final"]), as_f64(full["h_final"])) <= TOL["bf16"]


def test_gradient_carry_across_calls():
    # streaming a sequence in two calls: the second half's backward first (no dh_T), then the first
    # half's with dh_T = the second half's dh0; the gradients equal those of one call
    d = inputs.generate(1, 2, 2048, 64, 64, "bf16", 9, True, "weak")
    x = {n: d[n].cuda() for n in ("q", "k", "v", "g", "do")}
    half = lambda n, i: x[n][:, :, 1024 * i:1024 * (i + 1)].contiguous()
    fwd = gla.zeco_forward(x["q"], x["k"], x["v"], x["g"], 64, 2, 2)
    full = gla.zeco_backward(x["q"], x["k"], x["v"], x["g"], x["do"], fwd, 64, 2, 2)
    f1 = gla.zeco_forward(half("q", 0), half("k", 0), half("v", 0), half("g", 0), 64, 1, 1)
    f2 = gla.zeco_forward(half("q", 1), half("k", 1), half("v", 1), half("g", 1), 64, 1, 1, h0=f1["h_final"])
    b2 = gla.zeco_backward(half("q", 1), half("k", 1), half("v", 1), half("g", 1), half("do", 1), f2, 64, 1, 1)
    b1 = gla.zeco_backward(half("q", 0), half("k", 0), half("v", 0), half("g", 0), half("do", 0), f1, 64, 1, 1,
                           dhT=b2["dh0"])
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv", "dg"):
        got = torch.cat([b1[n], b2[n]], dim=2)
        assert maxrel(as_f64(got), as_f64(full[n])) <= TOL["bf16"], n
    assert maxrel(as_f64(b1["dh0"]), as_f64(full["dh0"])) <= TOL["bf16"]


def test_headline_workload_at_full_size():
    """64 segments of 16384 tokens, 4 heads, fwd+bwd, in the launch configuration the benchmark
    times, in both orders (the correction order, and the incoming states first with its state
    passes stopping where the decay ends).  The oracle runs head 0 in full, forward and backward
    over all 1M tokens, and every output and gradient of that head is compared element by element
    on every segment, for both orders; G[61] is checked against the oracle's backward over the last
    two segments.  The homogeneity identity sum<dq,q> = sum<dk,k> = sum<dv,v> = sum<do,o> is
    checked on every head, and the two orders agree on every head."""
    w = inputs.WORKLOADS[inputs.HEADLINE]
    t = time.time()
    d = inputs.generate_workload(w)
    say("generated %s in %.1fs" % (w.name, time.time() - t))
    x = dev(d)
    del d
    f = gla.zeco_forward(x["q"], x["k"], x["v"], x["g"], w.chunk, w.P, w.K)
    b = gla.zeco_backward(x["q"], x["k"], x["v"], x["g"], x["do"], f, w.chunk, w.P, w.K)
    sf = gla.states_first_forward(x["q"], x["k"], x["v"], x["g"], w.chunk, w.P, w.K)
    sb = gla.states_first_backward(x["q"], x["k"], x["v"], x["g"], x["do"], sf, w.chunk, w.K)
    torch.cuda.synchronize()
    assert sf["P"] == w.P
    say("gpu fwd+bwd done, both orders")
    both = {}
    for n, a_, b_ in (("o", sf["o"], f["o"]), ("h_final", sf["h_final"], f["h_final"]),
                      ("S_in", sf["seg_in"], f["seg_in"]), ("G", sb["seg_grad"], b["seg_grad"]),
                      ("dh0", sb["dh0"], b["dh0"]), ("dq", sb["dq"], b["dq"]), ("dk", sb["dk"], b["dk"]),
                      ("dv", sb["dv"], b["dv"]), ("dg", sb["dg"], b["dg"])):
        both[n] = float((a_.float() - b_.float()).abs().max() / b_.float().abs().max())
    say("states first against the correction order, every head: " + " ".join("%s=%.2e" % kv for kv in both.items()))
    assert max(both.values()) <= TOL["bf16"], both
    # homogeneity on every (b, h)
    ref = (x["do"].double() * f["o"].double()).sum(dim=(2, 3))
    for xn, dn in (("q", "dq"), ("k", "dk"), ("v", "dv")):
        gated, cond = homogeneity(x[xn], b[dn], ref)
        say("homogeneity %s: %.2e (over |sum<do,o>|: %.2e)" % (xn, max(gated), max(cond)))
        assert max(gated) <= TOL["bf16"], xn
    # oracle on head 0, every token
    h = inputs.generate_head(w.B, w.H, w.T, w.dk, w.dv, 0, 0, w.dtype, 0, True)
    a = {n: as_f64(t) for n, t in h.items()}
    del h
    L = w.L
    t62 = (w.P - 2) * L
    t = time.time()
    o_ref, hT, hs = oracle.gla_fwd(a["q"], a["k"], a["v"], a["g"], states_every=L)
    S62 = hs[:, :, w.P - 3]  # the state after 62 segments
    del hs
    say("oracle forward over %d tokens: %.1fs" % (w.T, time.time() - t))
    errs, el = {}, {}

    def cmp(name, got, r):
        errs[name] = maxrel(got, r)
        el[name] = elemrel(got, r)

    cmp("o", as_f64(f["o"][:1, :1]), o_ref)
    cmp("o (states first)", as_f64(sf["o"][:1, :1]), o_ref)
    del o_ref
    cmp("h_final", as_f64(f["h_final"][:1, :1]), hT)
    cmp("S_in[62]", as_f64(f["seg_in"][:1, :1, w.P - 2]), S62)
    cmp("S_in[62] (states first)", as_f64(sf["seg_in"][:1, :1, w.P - 2]), S62)
    t = time.time()
    gb = oracle.gla_bwd(a["q"], a["k"], a["v"], a["g"], a["do"])
    say("oracle backward over %d tokens: %.1fs" % (w.T, time.time() - t))
    for n in ("dq", "dk", "dv", "dg"):
        for tag, res in (("", b), (" (states first)", sb)):
            got = as_f64(res[n][:1, :1])
            cmp(n + tag, got, gb[n])
            # and segment by segment, so that no segment's error hides behind a larger one elsewhere
            seg = max(maxrel(got[:, :, p * L:(p + 1) * L], gb[n][:, :, p * L:(p + 1) * L]) for p in range(w.P))
            errs[n + tag + "[worst segment]"] = seg
            del got
    cmp("dh0", as_f64(b["dh0"][:1, :1]), gb["dh0"])
    cmp("dh0 (states first)", as_f64(sb["dh0"][:1, :1]), gb["dh0"])
    del gb
    gb2 = oracle.gla_bwd(a["q"][:, :, t62:], a["k"][:, :, t62:], a["v"][:, :, t62:], a["g"][:, :, t62:],
                         a["do"][:, :, t62:], S62)
    cmp("G[61]", as_f64(b["seg_grad"][:1, :1, w.P - 3]), gb2["dh0"])
    cmp("G[61] (states first)", as_f64(sb["seg_grad"][:1, :1, w.P - 3]), gb2["dh0"])
    say("headline workload, head 0, every token: " +
        " ".join("%s=%.2e" % kv for kv in errs.items()) + " | element-wise: " +
        " ".join("%s=%.1e" % kv for kv in el.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL["bf16"]}
    assert not bad, bad


@pytest.mark.parametrize("strong", [False, True], ids=["default-gates", "strong-stretches"])
def test_the_whole_path_replays_in_a_hip_graph(strong):
    """The six calls recorded into one HIP graph (torch's capture: no call allocates, clears or
    synchronises), replayed three times with eager work and synchronisations in between: every
    replay equals the eager run bit for bit.  16 heads of 8 segments, cut into sub-segments; with
    strong stretches the fast kernels flag units and the re-split redoes them, inside the graph."""
    B, H, T, dk, dv, chunk, P, K = 1, 16, 65536, 64, 64, 64, 8, 2
    d = inputs.generate(B, H, T, dk, dv, "bf16", 31, True, "logsigmoid16")
    if strong:
        d["g"] = inputs.add_strong_windows(d["g"], P, 12)
    x = dev(d)
    ws = torch.empty(gla.workspace_size(gla.GLA_BWD, B, H, T, dk, dv, chunk, P, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    f32 = dict(device="cuda", dtype=torch.float32)
    buf = {"o": torch.empty_like(x["v"]), "cs": torch.empty((B, H, T // chunk, dk, dv), device="cuda",
                                                             dtype=torch.bfloat16),
           "S": torch.empty((B, H, P, dk, dv), **f32), "ld": torch.empty((B, H, P, dk), **f32),
           "S_in": torch.empty((B, H, P, dk, dv), **f32), "h": torch.empty((B, H, dk, dv), **f32),
           "dq": torch.empty_like(x["q"]), "dk": torch.empty_like(x["k"]), "dv": torch.empty_like(x["v"]),
           "dg": torch.empty_like(x["g"]), "D": torch.empty((B, H, P, dk, dv), **f32),
           "G": torch.empty((B, H, P, dk, dv), **f32), "dh0": torch.empty((B, H, dk, dv), **f32)}
    q, k, v, g, do = x["q"], x["k"], x["v"], x["g"], x["do"]

    def path():
        gla.gla_chunk_fwd(q, k, v, g, chunk, P, o=buf["o"], chunk_states=buf["cs"], seg_state=buf["S"],
                          seg_logdecay=buf["ld"], workspace=ws)
        gla.gla_segment_scan(buf["S"], buf["ld"], K, seg_carry=buf["S_in"], h_out=buf["h"])
        gla.gla_segment_correct(gla.GLA_FWD, chunk, P, q=q, g=g, seg_in=buf["S_in"], o=buf["o"],
                                chunk_states=buf["cs"])
        gla.gla_chunk_bwd(q, k, v, g, do, buf["cs"], buf["S_in"], chunk, P, dq=buf["dq"], dk=buf["dk"],
                          dv=buf["dv"], dg=buf["dg"], seg_dstate=buf["D"], workspace=ws)
        gla.gla_segment_scan(buf["D"], buf["ld"], K, reverse=True, seg_carry=buf["G"], h_out=buf["dh0"])
        gla.gla_segment_correct(gla.GLA_BWD, chunk, P, k=k, v=v, g=g, seg_in=buf["S_in"], seg_grad=buf["G"],
                                chunk_states=buf["cs"], dk=buf["dk"], dv=buf["dv"], dg=buf["dg"])

    _replays_bit_for_bit(path, buf)
    check({n: as_f64(buf[n]) for n in ("o", "dq", "dk", "dv", "dg")},
          oracle_pipeline(d, chunk, P, True), ("o", "dq", "dk", "dv", "dg"), TOL["bf16"], "graph replay")


def _replays_bit_for_bit(path, buf):
    """Run path eagerly, record it into a HIP graph (after a warm-up on the capture's stream) and
    replay it three times with eager work and synchronisations in between: every replay must
    reproduce the eager run's buffers bit for bit."""
    path()
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in buf.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()  # warm-up on the capture's stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    torch.cuda.synchronize()
    for r in range(3):
        for t in buf.values():
            t.fill_(float("nan"))  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, t in ref.items():
            assert torch.equal(buf[n], t), (r, n)


def test_the_states_first_path_replays_in_a_hip_graph():
    """The order with the incoming states first recorded into one HIP graph: its state passes (cut
    into sub-segments here, each walking from its far end and stopping where the decay ends), the
    scans and the two local passes from the true incoming states; every replay equals the eager run
    bit for bit, and the results match the oracle."""
    B, H, T, dk, dv, chunk, P, K = 1, 16, 65536, 64, 64, 64, 8, 2
    d = inputs.generate(B, H, T, dk, dv, "bf16", 37, True, "logsigmoid16")
    x = dev(d)
    ws = torch.empty(gla.workspace_size(gla.GLA_BWD, B, H, T, dk, dv, chunk, P, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    f32 = dict(device="cuda", dtype=torch.float32)
    buf = {"o": torch.empty_like(x["v"]), "cs": torch.empty((B, H, T // chunk, dk, dv), device="cuda",
                                                             dtype=torch.bfloat16),
           "S": torch.empty((B, H, P, dk, dv), **f32), "ld": torch.empty((B, H, P, dk), **f32),
           "S_in": torch.empty((B, H, P, dk, dv), **f32), "h": torch.empty((B, H, dk, dv), **f32),
           "dq": torch.empty_like(x["q"]), "dk": torch.empty_like(x["k"]), "dv": torch.empty_like(x["v"]),
           "dg": torch.empty_like(x["g"]), "D": torch.empty((B, H, P, dk, dv), **f32),
           "G": torch.empty((B, H, P, dk, dv), **f32), "dh0": torch.empty((B, H, dk, dv), **f32)}
    q, k, v, g, do = x["q"], x["k"], x["v"], x["g"], x["do"]

    def path():
        gla.gla_chunk_state(k, v, g, chunk, P, seg_state=buf["S"], seg_logdecay=buf["ld"], workspace=ws)
        gla.gla_segment_scan(buf["S"], buf["ld"], K, seg_carry=buf["S_in"], h_out=buf["h"])
        gla.gla_chunk_fwd_from(q, k, v, g, buf["S_in"], chunk, P, o=buf["o"], chunk_states=buf["cs"], workspace=ws)
        gla.gla_chunk_dstate(q, g, do, chunk, P, seg_dstate=buf["D"], workspace=ws)
        gla.gla_segment_scan(buf["D"], buf["ld"], K, reverse=True, seg_carry=buf["G"], h_out=buf["dh0"])
        gla.gla_chunk_bwd_from(q, k, v, g, do, buf["cs"], buf["S_in"], buf["G"], chunk, P, dq=buf["dq"],
                               dk=buf["dk"], dv=buf["dv"], dg=buf["dg"], workspace=ws)

    _replays_bit_for_bit(path, buf)
    keys = ("o", "h", "dq", "dk", "dv", "dg", "dh0")
    gpu = {n: as_f64(buf[n]) for n in keys}
    ref = oracle_pipeline(d, chunk, P, True)
    ref["h"] = ref["h_final"]
    check(gpu, ref, keys, TOL["bf16"], "states-first graph replay")


def test_element_offsets_beyond_two_to_the_31():
    """9 heads of 1M tokens at d_k = 128, d_v = 256 (576 units, three waves of workgroups): v, o, do
    and dv hold 2.4e9 elements and the chunk states 4.8e9, so every kernel indexes past 2^31.  The
    last head, whose elements sit highest, is compared with the oracle over all its tokens; the
    homogeneity identity is checked on every head."""
    import dataclasses
    w = dataclasses.replace(inputs.WORKLOADS[inputs.HEADLINE], name="h9_t1m_p64", H=9)
    assert w.B * w.H * w.T * w.dv > 2 ** 31 and w.B * w.H * (w.T // w.chunk) * w.dk * w.dv > 2 ** 32
    t = time.time()
    x = dev(inputs.generate_workload(w))
    say("generated %s in %.1fs" % (w.name, time.time() - t))
    f = gla.zeco_forward(x["q"], x["k"], x["v"], x["g"], w.chunk, w.P, w.K)
    b = gla.zeco_backward(x["q"], x["k"], x["v"], x["g"], x["do"], f, w.chunk, w.P, w.K)
    torch.cuda.synchronize()
    say("gpu fwd+bwd done")

    ref = (x["do"].double() * f["o"].double()).sum(dim=(2, 3))
    hom = {}
    for xn, dn in (("q", "dq"), ("k", "dk"), ("v", "dv")):
        gated, cond = homogeneity(x[xn], b[dn], ref)
        say("homogeneity %s per head: %s (over |sum<do,o>|: %s)" % (xn, " ".join("%.1e" % r for r in gated),
                                                                   " ".join("%.1e" % r for r in cond)))
        hom[xn] = max(gated)
    hl = w.H - 1
    h = inputs.generate_head(w.B, w.H, w.T, w.dk, w.dv, 0, hl, w.dtype, 0, True)
    a = {n: as_f64(t_) for n, t_ in h.items()}
    del h
    t = time.time()
    o_ref, hT = oracle.gla_fwd(a["q"], a["k"], a["v"], a["g"])
    gb = oracle.gla_bwd(a["q"], a["k"], a["v"], a["g"], a["do"])
    say("oracle fwd+bwd of head %d over %d tokens: %.1fs" % (hl, w.T, time.time() - t))
    errs = {"o": maxrel(as_f64(f["o"][:1, hl:hl + 1]), o_ref), "h_final": maxrel(as_f64(f["h_final"][:1, hl:hl + 1]), hT)}
    for n in ("dq", "dk", "dv", "dg", "dh0"):
        errs[n] = maxrel(as_f64(b[n][:1, hl:hl + 1]), gb[n])
    say("head %d: " % hl + " ".join("%s=%.2e" % kv for kv in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL["bf16"]}
    assert not bad, bad
    assert all(r <= TOL["bf16"] for r in hom.values()), hom


@pytest.mark.parametrize("T_real,chunk,P", [(1000, 64, 4), (333, 16, 3), (4097, 32, 8)])
def test_a_ragged_sequence_padded_with_zeros_is_exact(T_real, chunk, P):
    """The calls take T as a multiple of P * chunk.  A sequence of any other length is padded at
    its end with q = k = v = do = 0 and g = 0: the padded tokens add nothing to the state and
    decay nothing, so the real tokens' outputs and gradients, h_final and dh0 are those of the
    unpadded sequence.  Checked against the oracle's recurrence over the T_real tokens alone,
    with boundary states."""
    B, H, dk, dv, K = 1, 2, 64, 128, 2
    step = P * chunk
    T = -(-T_real // step) * step
    d = inputs.generate(B, H, T_real, dk, dv, "bf16", 37, True, "logsigmoid16")
    pad = {}
    for n, t in d.items():
        z = torch.zeros((B, H, T - T_real, t.shape[-1]), dtype=t.dtype)
        pad[n] = torch.cat([t, z], dim=2).contiguous()
    rng = np.random.default_rng(5)
    h0 = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3)
    dhT = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.3)
    x = dev(pad)
    f = gla.zeco_forward(x["q"], x["k"], x["v"], x["g"], chunk, P, K, h0=h0.cuda())
    b = gla.zeco_backward(x["q"], x["k"], x["v"], x["g"], x["do"], f, chunk, P, K, dhT=dhT.cuda())
    torch.cuda.synchronize()
    a = {n: as_f64(t) for n, t in d.items()}
    o, hT = oracle.gla_fwd(a["q"], a["k"], a["v"], a["g"], h0.numpy())
    ref = {"o": o, "h_final": hT}
    ref.update(oracle.gla_bwd(a["q"], a["k"], a["v"], a["g"], a["do"], h0.numpy(), dhT.numpy()))
    got = {n: as_f64(f[n][:, :, :T_real]) for n in ("o",)}
    got["h_final"] = as_f64(f["h_final"])
    for n in ("dq", "dk", "dv", "dg"):
        got[n] = as_f64(b[n][:, :, :T_real])
    got["dh0"] = as_f64(b["dh0"])
    check(got, ref, ("o", "h_final", "dq", "dk", "dv", "dg", "dh0"), TOL["bf16"],
          "T %d padded to %d, chunk %d, P %d" % (T_real, T, chunk, P))
