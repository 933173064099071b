#!/usr/bin/env python
"""Benchmark: chunkwise GLA forward + backward with ZeCO's segment decomposition on one GPU.

One step = the whole path on one batch: gla_chunk_fwd -> gla_segment_scan -> gla_segment_correct
(forward), then gla_chunk_bwd -> gla_segment_scan(reverse) -> gla_segment_correct (backward).
Inputs are drawn once (seeded, synthetic) and stay resident in HBM; every output and intermediate
buffer is allocated before the timed region.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--gate VARIANT]
                  [--strong-windows N] [--no-cpu-baseline] [--no-extras] [--copy-calibration]
                  [--compare-orderings]

Besides the headline line, the default run adds (under "extras"): the same step with g = 0 (no
decay, so the corrections never stop early: the full second pass); the same step with 1, 8 and 32
strongly decaying 64-token stretches in as many segments (those segments take the exact kernels,
cut into pieces); the two-stream schedule; and the other fwd+bwd and forward workloads, each timed
over 50 iterations with a 512 MiB scrub written between them (untimed) so that no input stays in
the 256 MB last-level cache.  --strong-windows N puts N such stretches into the timed step itself.

--compare-orderings also times, on the same inputs, the two baseline orderings of the pages
rendered on one GPU, and adds them under "orderings": the all-gather scan (LASP2's pattern,
gla_segment_scan_allgather in place of the chain) and the serial chain (LASP1's pattern: no
segment runs before the previous one is done, i.e. the recurrence over the whole sequence, P = 1).

The roofline's "traffic" is the HBM bytes per launch of the dominant call as read by rocprofv3
counters (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a device copy of
known size); it is taken from profiles/<call>_<workload>_traffic.md and reported only while the
kernel sources still hash to the value recorded there (null otherwise).
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GLA fwd+bwd tokens/sec at 16k-token segments on 1 MI355X; % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


CSRC = os.path.join(ROOT, "sequence_state_scan_amd", "csrc")
# the sources that build each call's kernels (their hash dates a traffic measurement)
CALL_SOURCES = {
    "gla_chunk_fwd": ["gla_fwd.hip", "gla_exact.hip", "gla_common.hpp", "gla_kernels.hpp"],
    "gla_chunk_bwd": ["gla_bwd.hip", "gla_exact.hip", "gla_common.hpp", "gla_kernels.hpp"],
}
COPY_CALIBRATION_BYTES = 1 << 30
KERNELS_OF = {"gla_chunk_bwd": " (bwd_kernel)", "gla_chunk_fwd": " (fwd_local_kernel)"}


def sources_hash(call):
    h = hashlib.sha256()
    for f in CALL_SOURCES.get(call, []):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(call, workload):
    """HBM bytes per launch from the committed counter summary, if it still matches the sources."""
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.md" % (call, workload))
    if call not in CALL_SOURCES or not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    m_h = re.search(r"^sources_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not (m_b and m_h) or m_h.group(1) != sources_hash(call):
        return None
    return int(m_b.group(1))


def measured_mfma_busy(call, workload):
    """MFMA busy fraction of the call's main kernel from the committed counter summary, if it still
    matches the sources (null otherwise)."""
    path = os.path.join(ROOT, "profiles", "mfma_%s.md" % workload)
    if call not in CALL_SOURCES or not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"^mfma_busy_%s:\s*([0-9.]+)" % call, text, re.M)
    m_h = re.search(r"^sources_sha256_%s:\s*([0-9a-f]{64})" % call, text, re.M)
    if not (m_b and m_h) or m_h.group(1) != sources_hash(call):
        return None
    return float(m_b.group(1))


def alg_bytes(w, part):
    """Algorithmic HBM bytes: every input read once, every output written once (element size e
    for q/k/v/o/do/dq/dk/dv, 4 bytes for g/dg), plus the per-segment float32 states."""
    e = 2 if w.dtype == "bf16" else 4
    th = w.B * w.H * w.T
    units = w.B * w.H * w.P
    st = 4 * w.dk * w.dv
    if part == "fwd":          # q, k, v, g in; o out; segment states out/in/out
        return th * (e * (2 * w.dk + w.dv) + 4 * w.dk + e * w.dv) + units * st * 3
    if part == "chunk_bwd":    # q, k, v, g, do in; dq, dk, dv, dg out; seg_in in, D out
        return th * (e * (2 * w.dk + 2 * w.dv) + 4 * w.dk + e * (2 * w.dk + w.dv) + 4 * w.dk) + units * st * 2
    if part == "bwd":          # the whole backward: chunk_bwd plus the reverse scan's states
        return alg_bytes(w, "chunk_bwd") + units * st * 2
    raise ValueError(part)


def alg_flops(w, part):
    """Algorithmic flops (the causal half of the intra-chunk products counted).  part: "fwd" and
    "bwd" are whole passes (local call plus correction); "chunk_fwd" and "chunk_bwd" the local
    calls alone, whose kernels do not run the corrections' 2 dk dv / 4 dk dv per token-head."""
    th = w.B * w.H * w.T
    C, dk, dv = w.chunk, w.dk, w.dv
    seg = w.P > 1
    per = {
        "chunk_fwd": (C + 1) * (dk + dv) + 4 * dk * dv,
        "chunk_bwd": (C + 1) * (3 * dk + 2 * dv) + 8 * dk * dv,
    }
    per["fwd"] = per["chunk_fwd"] + (2 * dk * dv if seg else 0)
    per["bwd"] = per["chunk_bwd"] + (4 * dk * dv if seg else 0)
    return th * per[part]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_rate(oracle, a, w, threads, budget_s, min_tokens):
    """Time the oracle's fwd+bwd on the first n tokens of one head, n grown until one run takes at
    least 2/3 of budget_s (or covers the head).  Returns (seconds, tokens)."""
    n = min_tokens
    while True:
        t1 = min(n, w.T)
        sl = {k: v[:, :, :t1] for k, v in a.items()}
        t0 = time.perf_counter()
        oracle.gla_fwd(sl["q"], sl["k"], sl["v"], sl["g"], threads=threads)
        oracle.gla_bwd(sl["q"], sl["k"], sl["v"], sl["g"], sl["do"], threads=threads)
        dt = time.perf_counter() - t0
        if dt >= budget_s * 2 / 3 or t1 >= w.T:
            return dt, t1
        n = max(n + min_tokens, int(n * budget_s / max(dt, 1e-3)) // min_tokens * min_tokens)


def cpu_baseline(w, gate, budget_s=15.0, budget_1t_s=5.0):
    """The oracle (plain float64 recurrence, fwd+bwd) on a bounded sample of the workload: head 0,
    the first n tokens (whole segments), timed with every host thread and again with one."""
    import oracle
    from sequence_state_scan_amd import inputs
    from sequence_state_scan_amd.inputs import as_f64

    oracle.build(force=False)
    threads = oracle.max_threads()
    h = inputs.generate_head(w.B, w.H, w.T, w.dk, w.dv, 0, 0, w.dtype, 0, True, gate)
    a = {n: as_f64(t) for n, t in h.items()}
    spent, tokens = _oracle_rate(oracle, a, w, threads, budget_s, w.L)
    spent1, tokens1 = _oracle_rate(oracle, a, w, 1, budget_1t_s, min(w.L, 1024))
    # tokens of the workload per second: one head of `tokens` tokens is tokens / (B*H) workload tokens
    value = (tokens / (w.B * w.H)) / spent
    return {"value": value, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "value_1thread": (tokens1 / (w.B * w.H)) / spent1,
            "sample": "head 0 of %d, first %d tokens, fwd+bwd float64 token recurrence, %.2fs on %d threads "
                      "(1 thread: first %d tokens, %.2fs); value = tokens/(B*H)/time"
                      % (w.B * w.H, tokens, spent, threads, tokens1, spent1)}


def time_steps(torch, calls, steps, warmup, stream):
    """Warm up, then time `steps` passes over `calls` with events on the launch stream, twice: once
    with events around the whole timed region only (the step time: an event recorded between two
    calls leaves the GPU idle for about 10 us), then with events around every call (the per-call
    breakdown).  Returns (ms per step, mean ms per call, wall seconds of the first timed region)."""
    for _ in range(warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        for _, fn in calls:
            fn()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
          for _ in range(steps)]
    for s in range(steps):
        for i, (_, fn) in enumerate(calls):
            ev[s][i][0].record(stream)
            fn()
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    per_call = {name: sum(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)) / steps
                for i, (name, _) in enumerate(calls)}
    return start.elapsed_time(stop) / steps, per_call, wall


def compare_orderings(torch, gla, w, x, buf, stream, ms_chain, pc_chain):
    """The pages' baseline orderings on one GPU, same inputs and kernels: the all-gather scan in
    place of the chain, and the serial chain (P = 1: every chunk after the previous one)."""
    B, H, T, dk, dv, C, P, K = w.B, w.H, w.T, w.dk, w.dv, w.chunk, w.P, w.K
    q, k, v, g, do = x["q"], x["k"], x["v"], x["g"], x["do"]
    ag = [
        ("gla_segment_scan_allgather", lambda: gla.gla_segment_scan_allgather(buf["S_loc"], buf["ld"],
                                                                               seg_carry=buf["S_in"],
                                                                               h_out=buf["h_fin"])),
        ("gla_segment_scan_allgather(reverse)", lambda: gla.gla_segment_scan_allgather(
            buf["D"], buf["ld"], reverse=True, seg_carry=buf["G"], h_out=buf["dh0"])),
    ]
    ms_ag, pc_ag, _ = time_steps(torch, ag, 10, 2, stream)
    # serial chain: one segment per (b, h); the scan is a copy and the corrections find a zero
    # incoming state, so the step is the two local passes over the whole sequence.  A flags-only
    # workspace keeps each call from cutting the sequence into sub-segments (which would be the
    # decomposition again, inside the call)
    f32 = torch.float32
    one = {n: torch.empty((B, H, 1, dk, dv), device=q.device, dtype=f32) for n in ("S", "S_in", "D", "G")}
    ld1 = torch.empty((B, H, 1, dk), device=q.device, dtype=f32)
    ws1 = torch.empty(gla.flags_workspace_size(B, H, 1), device=q.device, dtype=torch.uint8)
    serial = [
        ("gla_chunk_fwd(P=1)", lambda: gla.gla_chunk_fwd(q, k, v, g, C, 1, o=buf["o"], chunk_states=buf["cs"],
                                                          seg_state=one["S"], seg_logdecay=ld1, workspace=ws1)),
        ("gla_segment_scan(P=1)", lambda: gla.gla_segment_scan(one["S"], ld1, K, seg_carry=one["S_in"],
                                                                h_out=buf["h_fin"])),
        ("gla_segment_correct(FWD, P=1)", lambda: gla.gla_segment_correct(gla.GLA_FWD, C, 1, q=q, g=g,
                                                                           seg_in=one["S_in"], o=buf["o"],
                                                                           chunk_states=buf["cs"])),
        ("gla_chunk_bwd(P=1)", lambda: gla.gla_chunk_bwd(q, k, v, g, do, buf["cs"], one["S_in"], C, 1,
                                                          dq=buf["dq"], dk=buf["dk"], dv=buf["dv"], dg=buf["dg"],
                                                          seg_dstate=one["D"], workspace=ws1)),
        ("gla_segment_scan(reverse, P=1)", lambda: gla.gla_segment_scan(one["D"], ld1, K, reverse=True,
                                                                         seg_carry=one["G"], h_out=buf["dh0"])),
        ("gla_segment_correct(BWD, P=1)", lambda: gla.gla_segment_correct(gla.GLA_BWD, C, 1, k=k, v=v, g=g,
                                                                           seg_in=one["S_in"], seg_grad=one["G"],
                                                                           chunk_states=buf["cs"], dk=buf["dk"],
                                                                           dv=buf["dv"], dg=buf["dg"])),
    ]
    ms_ser, pc_ser, _ = time_steps(torch, serial, 2, 1, stream)
    scans_chain = pc_chain["gla_segment_scan"] + pc_chain["gla_segment_scan(reverse)"]
    res = {
        "zeco_chain": {"ms_per_step": round(ms_chain, 4), "scan_ms": round(scans_chain, 4)},
        "allgather_scan": {"ms_per_step": round(ms_chain - scans_chain + ms_ag, 4), "scan_ms": round(ms_ag, 4),
                           "scan_calls_ms": {k_: round(v_, 4) for k_, v_ in pc_ag.items()}},
        "serial_chain_P1": {"ms_per_step": round(ms_ser, 4),
                            "per_call_ms": {k_: round(v_, 4) for k_, v_ in pc_ser.items()}},
    }
    log("orderings (ms per fwd+bwd step): ZeCO chain scan %.3f | all-gather scan %.3f (scans %.3f vs %.3f) | "
        "serial chain P=1 %.1f" % (ms_chain, res["allgather_scan"]["ms_per_step"], ms_ag, scans_chain, ms_ser))
    return res


def path_buffers(torch, gla, w, dev, edt, bwd=True, P=None):
    """Every output and intermediate of one fwd+bwd step, and the two calls' workspaces, allocated
    before anything is timed.  A forward-only workload keeps no per-chunk states (they exist for
    the backward only).  P: the segment count the per-segment buffers are sized for (default: the
    workload's)."""
    B, H, T, dk, dv, C = w.B, w.H, w.T, w.dk, w.dv, w.chunk
    P = w.P if P is None else P
    f32 = torch.float32
    st = (B, H, P, dk, dv)
    ws = max(gla.workspace_size(gla.GLA_FWD, B, H, T, dk, dv, C, P, edt),
             gla.workspace_size(gla.GLA_BWD, B, H, T, dk, dv, C, P, edt))
    return {
        "o": torch.empty((B, H, T, dv), device=dev, dtype=edt),
        "cs": torch.empty((B, H, T // C, dk, dv), device=dev, dtype=edt) if bwd else None,
        "S_loc": torch.empty(st, device=dev, dtype=f32), "ld": torch.empty((B, H, P, dk), device=dev, dtype=f32),
        "S_in": torch.empty(st, device=dev, dtype=f32), "h_fin": torch.empty((B, H, dk, dv), device=dev, dtype=f32),
        "dq": torch.empty((B, H, T, dk), device=dev, dtype=edt), "dk": torch.empty((B, H, T, dk), device=dev, dtype=edt),
        "dv": torch.empty((B, H, T, dv), device=dev, dtype=edt), "dg": torch.empty((B, H, T, dk), device=dev, dtype=f32),
        "D": torch.empty(st, device=dev, dtype=f32), "G": torch.empty(st, device=dev, dtype=f32),
        "dh0": torch.empty((B, H, dk, dv), device=dev, dtype=f32),
        "ws": torch.empty(ws, device=dev, dtype=torch.uint8), "P": P,
    }


def path_calls(gla, w, x, buf, bwd=True):
    """The calls of one step: the forward chain, and with bwd the backward chain."""
    C, P, K = w.chunk, w.P, w.K
    q, k, v, g = x["q"], x["k"], x["v"], x["g"]
    calls = [
        ("gla_chunk_fwd", lambda: gla.gla_chunk_fwd(q, k, v, g, C, P, o=buf["o"], chunk_states=buf["cs"],
                                                     seg_state=buf["S_loc"], seg_logdecay=buf["ld"],
                                                     workspace=buf["ws"], keep_chunk_states=buf["cs"] is not None)),
        ("gla_segment_scan", lambda: gla.gla_segment_scan(buf["S_loc"], buf["ld"], K, seg_carry=buf["S_in"],
                                                           h_out=buf["h_fin"])),
        ("gla_segment_correct(FWD)", lambda: gla.gla_segment_correct(gla.GLA_FWD, C, P, q=q, g=g, seg_in=buf["S_in"],
                                                                      o=buf["o"], chunk_states=buf["cs"])),
    ]
    if bwd:
        do = x["do"]
        calls += [
            ("gla_chunk_bwd", lambda: gla.gla_chunk_bwd(q, k, v, g, do, buf["cs"], buf["S_in"], C, P, dq=buf["dq"],
                                                         dk=buf["dk"], dv=buf["dv"], dg=buf["dg"], seg_dstate=buf["D"],
                                                         workspace=buf["ws"])),
            ("gla_segment_scan(reverse)", lambda: gla.gla_segment_scan(buf["D"], buf["ld"], K, reverse=True,
                                                                        seg_carry=buf["G"], h_out=buf["dh0"])),
            ("gla_segment_correct(BWD)", lambda: gla.gla_segment_correct(gla.GLA_BWD, C, P, k=k, v=v, g=g,
                                                                          seg_in=buf["S_in"], seg_grad=buf["G"],
                                                                          chunk_states=buf["cs"], dk=buf["dk"],
                                                                          dv=buf["dv"], dg=buf["dg"])),
        ]
    return calls


def states_first_buffers(torch, gla, w, buf):
    """buf with its per-segment buffers sized for the segment count of the order with the incoming
    states first (gla.states_first_segments: the workload's segments cut to fill the chip)."""
    P = gla.states_first_segments(w.B, w.H, w.T, w.chunk, w.P)
    if P == buf["P"]:
        return buf
    out = dict(buf, P=P)
    for n in ("S_loc", "S_in", "D", "G"):
        out[n] = torch.empty((w.B, w.H, P, w.dk, w.dv), device=buf["o"].device, dtype=torch.float32)
    out["ld"] = torch.empty((w.B, w.H, P, w.dk), device=buf["o"].device, dtype=torch.float32)
    return out


def path_calls_states_first(gla, w, x, buf, bwd=True):
    """The same step with the segments' incoming states first: state pass, scan, local pass from the
    true incoming state (no correction), and with bwd the same for the backward, over the
    buffers' segment count (path_buffers with P = gla.states_first_segments(...): the segments cut
    to fill the chip)."""
    C, P, K = w.chunk, buf["P"], w.K
    q, k, v, g = x["q"], x["k"], x["v"], x["g"]
    calls = [
        ("gla_chunk_state", lambda: gla.gla_chunk_state(k, v, g, C, P, seg_state=buf["S_loc"], seg_logdecay=buf["ld"],
                                                         workspace=buf["ws"])),
        ("gla_segment_scan", lambda: gla.gla_segment_scan(buf["S_loc"], buf["ld"], K, seg_carry=buf["S_in"],
                                                           h_out=buf["h_fin"])),
        ("gla_chunk_fwd_from", lambda: gla.gla_chunk_fwd_from(q, k, v, g, buf["S_in"], C, P, o=buf["o"],
                                                               chunk_states=buf["cs"], workspace=buf["ws"],
                                                               keep_chunk_states=buf["cs"] is not None)),
    ]
    if not bwd:
        return calls
    do = x["do"]
    return calls + [
        ("gla_chunk_dstate", lambda: gla.gla_chunk_dstate(q, g, do, C, P, seg_dstate=buf["D"], workspace=buf["ws"])),
        ("gla_segment_scan(reverse)", lambda: gla.gla_segment_scan(buf["D"], buf["ld"], K, reverse=True,
                                                                    seg_carry=buf["G"], h_out=buf["dh0"])),
        ("gla_chunk_bwd_from", lambda: gla.gla_chunk_bwd_from(q, k, v, g, do, buf["cs"], buf["S_in"], buf["G"], C, P,
                                                               dq=buf["dq"], dk=buf["dk"], dv=buf["dv"], dg=buf["dg"],
                                                               workspace=buf["ws"])),
    ]


def time_scrubbed(torch, calls, iters, warmup, stream, scrub):
    """Time each of `iters` steps on its own, with `scrub` (a large buffer) overwritten between them
    outside the timed events, so that no input is left in the last-level cache.  Returns
    (mean ms, median ms, mean ms per call)."""
    for _ in range(warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
          for _ in range(iters)]
    for it in range(iters):
        scrub.add_(1)
        for i, (_, fn) in enumerate(calls):
            ev[it][i][0].record(stream)
            fn()
            ev[it][i][1].record(stream)
    torch.cuda.synchronize()
    steps = sorted(sum(ev[it][i][0].elapsed_time(ev[it][i][1]) for i in range(len(calls))) for it in range(iters))
    per_call = {name: sum(ev[it][i][0].elapsed_time(ev[it][i][1]) for it in range(iters)) / iters
                for i, (name, _) in enumerate(calls)}
    return sum(steps) / iters, steps[iters // 2], per_call


def other_workloads(torch, gla, inputs, dev, stream, names, iters=50, warmup=5):
    """The remaining fwd+bwd and forward workloads at full size, each step timed alone with a
    512 MiB scrub between steps."""
    scrub = torch.zeros(128 << 20, dtype=torch.float32, device=dev)  # 512 MiB
    out = {}
    for name in names:
        w = inputs.WORKLOADS[name]
        d = inputs.generate_workload(w, bwd=w.bwd)
        x = {n: t.to(dev) for n, t in d.items()}
        del d
        buf = path_buffers(torch, gla, w, dev, x["q"].dtype, bwd=w.bwd)
        calls = path_calls(gla, w, x, buf, bwd=w.bwd)
        mean, med, per_call = time_scrubbed(torch, calls, iters, warmup, stream, scrub)
        ab = alg_bytes(w, "fwd") + (alg_bytes(w, "bwd") if w.bwd else 0)
        af = alg_flops(w, "fwd") + (alg_flops(w, "bwd") if w.bwd else 0)
        out[name] = {
            "pass": "fwd+bwd" if w.bwd else "fwd", "chunk_states_kept": bool(w.bwd),
            "tokens_per_s": round(w.B * w.T / (mean / 1e3), 1),
            "ms_mean": round(mean, 4), "ms_median": round(med, 4), "iters": iters,
            "hbm_frac": round(ab / (mean / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(af / (mean / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4), "alg_bytes": ab,
            "per_call_ms": {k_: round(v_, 4) for k_, v_ in per_call.items()},
        }
        log("%s: %.4f ms mean (%.4f median), %.3f of HBM peak" % (name, mean, med, out[name]["hbm_frac"]))
        # the same step with the incoming states first (no correction pass)
        sbuf = states_first_buffers(torch, gla, w, buf)
        mean, med, per_call = time_scrubbed(torch, path_calls_states_first(gla, w, x, sbuf, bwd=w.bwd), iters, warmup,
                                            stream, scrub)
        out[name]["states_first"] = {
            "segments": sbuf["P"],
            "tokens_per_s": round(w.B * w.T / (mean / 1e3), 1), "ms_mean": round(mean, 4), "ms_median": round(med, 4),
            "hbm_frac": round(ab / (mean / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "per_call_ms": {k_: round(v_, 4) for k_, v_ in per_call.items()},
        }
        log("%s, states first: %.4f ms mean, %.3f of HBM peak" % (name, mean, out[name]["states_first"]["hbm_frac"]))
        del x, buf, sbuf, calls
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--gate", default="logsigmoid16")
    ap.add_argument("--strong-windows", type=int, default=0,
                    help="add this many strongly decaying 64-token stretches to the gates, in as many segments")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline step (no g = 0 step, no other workloads)")
    ap.add_argument("--order", choices=("correction", "states-first"), default="correction",
                    help="the order of the step's calls: local pass, scan, correction (ZeCO's), or state pass, "
                         "scan, local pass from the true incoming state")
    ap.add_argument("--streams", type=int, default=1,
                    help="time the step with the sequences split over this many streams (zeco_step_streams)")
    ap.add_argument("--stagger", action="store_true",
                    help="with --streams: each group waits for the previous group's local pass")
    ap.add_argument("--compare-orderings", action="store_true",
                    help="also time the all-gather scan and the serial chain (P = 1) on the same inputs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy %d bytes device to device (untimed), the reference for the byte counters"
                         % COPY_CALIBRATION_BYTES)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library runs every segment on a single MI355X and has no "
              "multi-GPU path; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from sequence_state_scan_amd import gla, inputs

    w = inputs.WORKLOADS[args.workload or inputs.HEADLINE]
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    gla.load_library()

    t = time.time()
    d = inputs.generate_workload(w, gate=args.gate, bwd=True)
    if args.strong_windows:
        d["g"] = inputs.add_strong_windows(d["g"], w.P, args.strong_windows)
    x = {n: v.to(dev) for n, v in d.items()}
    del d
    log("inputs %s drawn and uploaded in %.1fs" % (w.name, time.time() - t))

    B, H, T, dk, dv, C, P, K = w.B, w.H, w.T, w.dk, w.dv, w.chunk, w.P, w.K
    buf = path_buffers(torch, gla, w, dev, x["q"].dtype)
    calls = (path_calls(gla, w, x, buf) if args.order == "correction" else
             path_calls_states_first(gla, w, x, states_first_buffers(torch, gla, w, buf)))
    if args.streams > 1:
        sbuf = gla.zeco_step_streams(x["q"], x["k"], x["v"], x["g"], x["do"], C, P, K, args.streams)
        calls = [("zeco_step_streams(%d)" % args.streams,
                  lambda: gla.zeco_step_streams(x["q"], x["k"], x["v"], x["g"], x["do"], C, P, K, args.streams,
                                                out=sbuf, stagger=args.stagger))]

    if args.copy_calibration:
        src = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: %d bytes copied" % COPY_CALIBRATION_BYTES)

    stream = torch.cuda.current_stream(dev)  # the stream every call launches on
    ms_step, per_call, wall = time_steps(torch, calls, args.steps, args.warmup, stream)
    tokens = B * T
    value = tokens / (ms_step / 1e3)

    # the dominant call and its roofline (algorithmic bytes of that call / its mean duration)
    dom = max(per_call, key=per_call.get) if args.streams == 1 else None
    if dom in ("gla_chunk_bwd", "gla_chunk_bwd_from"):  # the same inputs and outputs
        dom_bytes, dom_flops = alg_bytes(w, "chunk_bwd"), alg_flops(w, "chunk_bwd")
    elif dom == "gla_chunk_fwd":
        dom_bytes, dom_flops = alg_bytes(w, "fwd"), alg_flops(w, "chunk_fwd")
    else:
        dom_bytes, dom_flops = None, None
    roof = None
    if dom_bytes:
        ach = dom_bytes / (per_call[dom] / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dom, w.name),
                "kernel": dom + KERNELS_OF.get(dom, ""),
                "alg_bytes_per_launch": dom_bytes,
                "mfma_frac": round(dom_flops / (per_call[dom] / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "mfma_busy_counter": measured_mfma_busy(dom, w.name)}
    step_bytes = alg_bytes(w, "fwd") + alg_bytes(w, "bwd")
    step_flops = alg_flops(w, "fwd") + alg_flops(w, "bwd")
    step_roof = {"alg_bytes": step_bytes, "hbm_frac": round(step_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                 "alg_flops": step_flops,
                 "mfma_frac": round(step_flops / (ms_step / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)}

    orderings = None
    if args.compare_orderings:
        orderings = compare_orderings(torch, gla, w, x, buf, stream, ms_step, per_call)

    extras = None
    if not args.no_extras and w.name == inputs.HEADLINE:
        # the same step with g = 0: no decay, so both corrections run over every chunk
        x0 = dict(x)
        x0["g"] = torch.zeros_like(x["g"])
        ms0, pc0, _ = time_steps(torch, path_calls(gla, w, x0, buf), 10, 3, stream)
        log("g = 0: %.4f ms per step" % ms0)
        # and in the order with the incoming states first, which has no correction pass to grow
        ms0s, pc0s, _ = time_steps(torch, path_calls_states_first(gla, w, x0, states_first_buffers(torch, gla, w, buf)),
                                   10, 3, stream)
        del x0
        log("g = 0, states first: %.4f ms per step" % ms0s)
        extras = {"no_decay_step": {
            "gate": "zero", "ms_per_step": round(ms0, 4), "tokens_per_s": round(tokens / (ms0 / 1e3), 1),
            "hbm_frac": round(step_bytes / (ms0 / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "per_call_ms": {k_: round(v_, 4) for k_, v_ in pc0.items()},
            "states_first": {"ms_per_step": round(ms0s, 4), "tokens_per_s": round(tokens / (ms0s / 1e3), 1),
                             "hbm_frac": round(step_bytes / (ms0s / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                             "per_call_ms": {k_: round(v_, 4) for k_, v_ in pc0s.items()}}}}
        # the headline step itself in that order (default gates)
        mss, pcs, _ = time_steps(torch, path_calls_states_first(gla, w, x, states_first_buffers(torch, gla, w, buf)),
                                 10, 3, stream)
        log("states first: %.4f ms per step" % mss)
        extras["states_first_step"] = {"gate": args.gate, "ms_per_step": round(mss, 4),
                                       "tokens_per_s": round(tokens / (mss / 1e3), 1),
                                       "per_call_ms": {k_: round(v_, 4) for k_, v_ in pcs.items()}}
        if args.strong_windows == 0 and args.gate == "logsigmoid16":
            # the same step with a few strongly decaying 64-token stretches: the segments they touch
            # are flagged by the fast kernels and redone, cut into pieces, by the exact kernels
            extras["strong_windows_steps"] = {}
            for n_w in (1, 8, 32):
                xw = dict(x, g=inputs.add_strong_windows(x["g"], P, n_w))
                msw, pcw, _ = time_steps(torch, path_calls(gla, w, xw, buf), 10, 3, stream)
                del xw
                log("%d strong windows: %.4f ms per step" % (n_w, msw))
                extras["strong_windows_steps"][str(n_w)] = {
                    "ms_per_step": round(msw, 4), "tokens_per_s": round(tokens / (msw / 1e3), 1),
                    "per_call_ms": {k_: round(v_, 4) for k_, v_ in pcw.items()}}
        if args.streams == 1:
            # the same step with the heads split over two streams (the scans and corrections of one
            # half can run beside the local passes of the other)
            sbuf = gla.zeco_step_streams(x["q"], x["k"], x["v"], x["g"], x["do"], C, P, K, 2)
            ms2, _, _ = time_steps(torch, [("two streams", lambda: gla.zeco_step_streams(
                x["q"], x["k"], x["v"], x["g"], x["do"], C, P, K, 2, out=sbuf))], 10, 3, stream)
            del sbuf
            log("two streams: %.4f ms per step" % ms2)
            extras["two_stream_step"] = {"ms_per_step": round(ms2, 4), "tokens_per_s": round(tokens / (ms2 / 1e3), 1)}
        del x, buf, calls
        torch.cuda.empty_cache()
        extras["workloads"] = other_workloads(torch, gla, inputs, dev, stream,
                                              [n for n in inputs.WORKLOADS if n != w.name and
                                               inputs.WORKLOADS[n].dtype == "bf16"])

    cpu = None
    if not args.no_cpu_baseline:
        t = time.time()
        cpu = cpu_baseline(w, args.gate)
        log("cpu baseline in %.1fs" % (time.time() - t))

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "chunk": C, "P": P, "K": K,
                   "segment_tokens": w.L, "gate": args.gate, "order": args.order, "streams": args.streams,
                   "stagger": bool(args.stagger)},
        "roofline": roof, "cpu_baseline": cpu,
        "step_roofline": step_roof,
        "per_call_ms": {k_: round(v_, 4) for k_, v_ in per_call.items()},
        "wall_s_timed": round(wall, 3),
    }
    if orderings is not None:
        out["orderings"] = orderings
    if extras is not None:
        out["extras"] = extras
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
