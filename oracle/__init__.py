"""Float64 CPU oracle for chunk-free gated linear attention and ZeCO's segment decomposition.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU path (no kernels, headers,
helpers or constants) and imports nothing from it.

Contents
--------
* ``gla_fwd`` / ``gla_bwd`` / ``gla_dg_direct``: the token-by-token recurrence and its backward,
  written in plain C (``gla_oracle.c``, float64) and called through ctypes.
* ``bruteforce_fwd``: the same forward as an explicit quadratic sum over (t, s, channel), in
  numpy.  It is one of the pins of ``gla_fwd``.
* ``segment_*``: ZeCO's linear decomposition, in float64 numpy, step by step:
  local pass from a zero state, decay-and-add scan over segments, cumulative-decay correction.
  The pages state the scan update ("What carries the argument" on the pith.science review of
  ZeCO: each rank applies S_p = (cumulative decay) * S_{p-1} + S_local on each of K row blocks)
  and the decomposition identity (same page, "Assumptions": the local recurrence can be run from
  a zero state and corrected by a cumulative decay, proved in the paper's Appendix A.1).  The
  backward's cross-segment gradient is not derived on the pages (same list: Appendix A.4 only
  says the forward's global state is reused); it is taken here as the same decay-and-add scan run
  in reverse over the state gradient.

Conventions: arrays are [B, H, T, d] (tokens-major per head), states [B, H, dk, dv], segment
arrays [B, H, P, ...].  Every function accepts any float dtype and works in float64.

Parity status: every function here is pinned by ``tests/test_oracle.py`` (brute force, textbook
special cases, finite differences, torch float64 autograd, the decomposition identity and scan
special cases); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_gla_oracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile ``gla_oracle.c`` into ``_gla_oracle.so`` with gcc (float64, OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            _lib = load_library(_LIB_PATH)
    return _lib


def load_library(path: str):
    """Open a compiled copy of ``gla_oracle.c`` and declare its C signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_gla_fwd.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp, i, i]
    lib.oracle_gla_fwd.restype = None
    lib.oracle_gla_bwd.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, i]
    lib.oracle_gla_bwd.restype = None
    lib.oracle_gla_dg_direct.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp, i]
    lib.oracle_gla_dg_direct.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def max_threads() -> int:
    """Threads the OpenMP runtime of the oracle library will use by default."""
    return int(_load().oracle_max_threads())


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _dims(q, v):
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    return B, H, T, dk, dv


# ----------------------------------------------------------------------------------------------
# Token recurrence (C)
# ----------------------------------------------------------------------------------------------

def gla_fwd(q, k, v, g, h0=None, threads: int = 0, states_every: int = 0):
    """Token-by-token forward.  Returns (o [B,H,T,dv], hT [B,H,dk,dv]), float64, and with
    states_every = C > 0 also the state after every C tokens, [B,H,T//C,dk,dv].

    S_t = diag(exp(g_t)) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, S_{-1} = h0 (zeros if None).
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, H, T, dk, dv = _dims(q, v)
    h0 = None if h0 is None else _f64(h0)
    o = np.empty((B, H, T, dv), dtype=np.float64)
    hT = np.empty((B, H, dk, dv), dtype=np.float64)
    hs = np.empty((B, H, T // states_every, dk, dv), dtype=np.float64) if states_every > 0 else None
    _load().oracle_gla_fwd(B * H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0),
                           _ptr(o), _ptr(hT), _ptr(hs), int(states_every), int(threads))
    if hs is not None:
        return o, hT, hs
    return o, hT


def gla_bwd(q, k, v, g, do, h0=None, dhT=None, threads: int = 0):
    """Token-by-token backward of L = sum <do, o> + <dhT, S_{T-1}>.

    Returns a dict with dq, dk, dv, dg ([B,H,T,*]) and dh0 ([B,H,dk,dv]), float64.  dg uses the
    closed form (reverse running sum of q*dq - k*dk plus rowsum(S_{T-1} * dhT)).
    """
    q, k, v, g, do = _f64(q), _f64(k), _f64(v), _f64(g), _f64(do)
    B, H, T, dk, dv = _dims(q, v)
    h0 = None if h0 is None else _f64(h0)
    dhT = None if dhT is None else _f64(dhT)
    dq = np.empty_like(q)
    dkk = np.empty_like(k)
    dvv = np.empty_like(v)
    dg = np.empty_like(g)
    dh0 = np.empty((B, H, dk, dv), dtype=np.float64)
    _load().oracle_gla_bwd(B * H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(do),
                           _ptr(h0), _ptr(dhT), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dg), _ptr(dh0),
                           int(threads))
    return {"dq": dq, "dk": dkk, "dv": dvv, "dg": dg, "dh0": dh0}


def gla_dg_direct(q, k, v, g, do, h0=None, dhT=None, threads: int = 0):
    """dg by its direct form exp(g_t) * <S_{t-1}[c,:], U_t[c,:]> (keeps a row history: small T)."""
    q, k, v, g, do = _f64(q), _f64(k), _f64(v), _f64(g), _f64(do)
    B, H, T, dk, dv = _dims(q, v)
    h0 = None if h0 is None else _f64(h0)
    dhT = None if dhT is None else _f64(dhT)
    dg = np.empty_like(g)
    rc = _load().oracle_gla_dg_direct(B * H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                      _ptr(do), _ptr(h0), _ptr(dhT), _ptr(dg), int(threads))
    if rc != 0:
        raise MemoryError("oracle_gla_dg_direct: out of memory")
    return dg


# ----------------------------------------------------------------------------------------------
# Quadratic closed form (numpy), small inputs only
# ----------------------------------------------------------------------------------------------

def bruteforce_fwd(q, k, v, g, h0=None):
    """o_t = sum_{s<=t} sum_c q_tc k_sc exp(B_tc - B_sc) v_s + sum_c q_tc exp(B_tc) h0[c,:].

    B_t = sum_{r<=t} g_r (running log-decay).  This is the recurrence unrolled; it is written
    independently of the C loops and costs O(T^2 dk dv).
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, H, T, dk, dv = _dims(q, v)
    Bc = np.cumsum(g, axis=2)  # [B,H,T,dk]
    o = np.zeros((B, H, T, dv))
    for t in range(T):
        w = np.exp(Bc[:, :, t:t + 1, :] - Bc[:, :, : t + 1, :])  # [B,H,t+1,dk]
        coef = np.einsum("bhc,bhsc->bhs", q[:, :, t, :], k[:, :, : t + 1, :] * w)
        o[:, :, t, :] = np.einsum("bhs,bhsj->bhj", coef, v[:, :, : t + 1, :])
        if h0 is not None:
            o[:, :, t, :] += np.einsum("bhc,bhcj->bhj", q[:, :, t, :] * np.exp(Bc[:, :, t, :]), _f64(h0))
    return o


# ----------------------------------------------------------------------------------------------
# ZeCO segment decomposition (numpy, float64)
# ----------------------------------------------------------------------------------------------

def _split(x, P):
    B, H, T = x.shape[:3]
    if T % P:
        raise ValueError("T=%d is not a multiple of P=%d" % (T, P))
    return x.reshape(B, H, P, T // P, *x.shape[3:])


def _merge(x):
    B, H, P, L = x.shape[:4]
    return x.reshape(B, H, P * L, *x.shape[4:])


def segment_local_fwd(q, k, v, g, P: int, threads: int = 0, chunk: int = 0):
    """Local pass: every segment from a zero state.

    Returns (o_local [B,H,T,dv], S_local [B,H,P,dk,dv], logdecay [B,H,P,dk]) where S_local is the
    segment's end state when it starts from zero and logdecay is the sum of g over the segment
    (the log of the cumulative decay the All-Scan update applies).  With chunk = C > 0 it also
    returns the local state after every C tokens, [B,H,T//C,dk,dv] (the chunk states the local
    pass stores).
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, H, T, dk, dv = _dims(q, v)
    qs, ks, vs, gs = (_split(x, P) for x in (q, k, v, g))
    L = T // P
    # Treat (B, H, P) as the batch of independent zero-state sequences.
    res = gla_fwd(qs.reshape(B * H * P, 1, L, dk), ks.reshape(B * H * P, 1, L, dk),
                  vs.reshape(B * H * P, 1, L, dv), gs.reshape(B * H * P, 1, L, dk), None, threads,
                  states_every=chunk)
    o_local = res[0].reshape(B, H, T, dv)
    S_local = res[1].reshape(B, H, P, dk, dv)
    logdecay = gs.sum(axis=3)
    if chunk > 0:
        return o_local, S_local, logdecay, res[2].reshape(B, H, T // chunk, dk, dv)
    return o_local, S_local, logdecay


def segment_scan(seg_state, logdecay, h_boundary=None, reverse: bool = False):
    """Decay-and-add scan over segments.

    Forward (reverse=False): carry[0] = h_boundary (h0), carry[p+1] = exp(logdecay[p]) * carry[p]
    + seg_state[p]; returns (carry [B,H,P,dk,dv] = state entering each segment, h_out = state
    after the last segment).

    Reverse (reverse=True): seg_state holds each segment's local state-gradient D_p; with
    G_{P-1} = h_boundary (dL/dS_T), G_{p-1} = exp(logdecay[p]) * G_p + D_p; returns
    (carry[p] = G_p = gradient w.r.t. the state leaving segment p, h_out = dh0 =
    exp(logdecay[0]) * G_0 + D_0).

    exp(logdecay) scales whole d_k rows, so splitting rows into blocks changes nothing.
    """
    S = _f64(seg_state)
    ld = _f64(logdecay)
    B, H, P, dk, dv = S.shape
    carry = np.empty_like(S)
    acc = np.zeros((B, H, dk, dv)) if h_boundary is None else _f64(h_boundary).copy()
    for p in (range(P - 1, -1, -1) if reverse else range(P)):
        carry[:, :, p] = acc
        acc = np.exp(ld[:, :, p])[..., None] * acc + S[:, :, p]
    return carry, acc


def segment_correct_fwd(o_local, q, g, seg_in, P: int, chunk_states_local=None, chunk: int = 0):
    """o_t = o_local_t + (q_t * a_t) . S_in[p],  a_t = exp(sum of g from the segment start to t).

    With the local chunk states (and their chunk length) it also returns the global ones:
    state after chunk n = local state after chunk n + diag(a at the chunk's last token) S_in[p].
    """
    o_local, q, g, S_in = _f64(o_local), _f64(q), _f64(g), _f64(seg_in)
    a = np.exp(np.cumsum(_split(g, P), axis=3))  # inclusive, within each segment
    corr = np.matmul(_split(q, P) * a, S_in)        # [..., L, dk] @ [..., dk, dv]
    o = o_local + _merge(corr)
    if chunk_states_local is None:
        return o
    B, H, Pn, L, dk = a.shape
    n_per = L // chunk
    a_end = a[:, :, :, chunk - 1::chunk, :]  # [B,H,P,n_per,dk]
    cs = _f64(chunk_states_local).reshape(B, H, Pn, n_per, dk, -1)
    cs = cs + a_end[..., None] * S_in[:, :, :, None, :, :]
    return o, cs.reshape(B, H, Pn * n_per, dk, -1)


def segment_local_bwd(q, k, v, g, do, seg_in, P: int, threads: int = 0):
    """Backward of every segment with its global incoming state and a zero terminal gradient.

    Returns dict(dq = global dq, dk_local, dv_local, dg_local, D_local [B,H,P,dk,dv]) where
    D_local[p] is the gradient w.r.t. the state entering segment p from segment p's own outputs.
    """
    q, k, v, g, do, S_in = _f64(q), _f64(k), _f64(v), _f64(g), _f64(do), _f64(seg_in)
    B, H, T, dk, dv = _dims(q, v)
    L = T // P
    r = lambda x, d: _split(x, P).reshape(B * H * P, 1, L, d)  # noqa: E731
    out = gla_bwd(r(q, dk), r(k, dk), r(v, dv), r(g, dk), r(do, dv),
                  S_in.reshape(B * H * P, 1, dk, dv), None, threads)
    return {
        "dq": out["dq"].reshape(B, H, T, dk),
        "dk_local": out["dk"].reshape(B, H, T, dk),
        "dv_local": out["dv"].reshape(B, H, T, dv),
        "dg_local": out["dg"].reshape(B, H, T, dk),
        "D_local": out["dh0"].reshape(B, H, P, dk, dv),
    }


def segment_correct_bwd(k, v, g, dk_local, dv_local, dg_local, seg_in, seg_grad, P: int,
                        h_final=None):
    """Add the later segments' state gradient G_p to every segment's local gradients.

    With r_t = sum of g over the tokens after t up to the segment end, e_t = exp(r_t):
      dk_t = dk_local_t + e_t * (G_p v_t)
      dv_t = dv_local_t + G_p^T (e_t * k_t)
      dg_t = dg_local_t - sum_{t' >= t in the segment} k_t' * (e_t' * (G_p v_t'))
             + rowsum(X_{p+1} * G_p)
    where X_{p+1} is the global state leaving segment p (seg_in[p+1], or h_final for the last
    segment; zero if h_final is None).
    """
    k, v, g = _f64(k), _f64(v), _f64(g)
    dk_local, dv_local, dg_local = _f64(dk_local), _f64(dv_local), _f64(dg_local)
    S_in, G = _f64(seg_in), _f64(seg_grad)
    B, H, T, dk, dv = _dims(k, v)
    gs = _split(g, P)
    rev_incl = np.flip(np.cumsum(np.flip(gs, axis=3), axis=3), axis=3)  # sum_{s>=t}
    r = np.zeros_like(gs)
    r[:, :, :, :-1, :] = rev_incl[:, :, :, 1:, :]  # sum_{s>t}
    e = np.exp(r)
    ks, vs = _split(k, P), _split(v, P)
    ddk = e * np.matmul(vs, np.swapaxes(G, -1, -2))  # (G v_t)[c]
    ddv = np.matmul(e * ks, G)                       # G^T (e_t k_t)
    X_next = np.zeros_like(S_in)
    X_next[:, :, :-1] = S_in[:, :, 1:]
    if h_final is not None:
        X_next[:, :, -1] = _f64(h_final)
    const = np.sum(X_next * G, axis=-1)  # [B,H,P,dk]
    kd = ks * ddk
    kd_suffix = np.flip(np.cumsum(np.flip(kd, axis=3), axis=3), axis=3)
    dg = _split(dg_local, P) - kd_suffix + const[:, :, :, None, :]
    return {
        "dk": dk_local + _merge(ddk),
        "dv": dv_local + _merge(ddv),
        "dg": _merge(dg),
    }


def zeco_fwd(q, k, v, g, P: int, h0=None, threads: int = 0, chunk: int = 0):
    """Forward through the decomposition: local pass, scan, correction.  Returns a dict; with
    chunk = C > 0 it holds the local and the corrected (global) state after every C tokens."""
    res = segment_local_fwd(q, k, v, g, P, threads, chunk)
    o_local, S_local, ld = res[:3]
    S_in, h_final = segment_scan(S_local, ld, h0, reverse=False)
    out = {"o_local": o_local, "S_local": S_local, "logdecay": ld, "S_in": S_in, "h_final": h_final}
    if chunk > 0:
        out["chunk_states_local"] = res[3]
        out["o"], out["chunk_states"] = segment_correct_fwd(o_local, q, g, S_in, P, res[3], chunk)
    else:
        out["o"] = segment_correct_fwd(o_local, q, g, S_in, P)
    return out


def zeco_bwd(q, k, v, g, do, P: int, S_in, logdecay, h_final=None, dhT=None, threads: int = 0):
    """Backward through the decomposition: local backward with the global incoming states,
    reverse scan of the local state-gradients, correction.  Returns a dict."""
    loc = segment_local_bwd(q, k, v, g, do, S_in, P, threads)
    G, dh0 = segment_scan(loc["D_local"], logdecay, dhT, reverse=True)
    fix = segment_correct_bwd(k, v, g, loc["dk_local"], loc["dv_local"], loc["dg_local"], S_in, G,
                              P, h_final)
    out = dict(loc)
    out.update(fix)
    out["G"] = G
    out["dh0"] = dh0
    return out
