"""Thin ctypes binding of libgla.so (C ABI in include/gla.h).

Argument marshalling only: every step runs in the HIP kernels of libgla.so.  torch provides
device memory (tensors) and the stream (torch's current stream on the tensors' device).
There is no CPU fallback: without the built library every call raises.

Low-level calls carry the C names (gla_chunk_fwd, gla_segment_scan, gla_segment_correct,
gla_chunk_bwd).  ``zeco_forward`` / ``zeco_backward`` chain them in the order of the method:
local pass -> segment scan -> correction, and the same for the backward.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgla.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "gla.h")

GLA_OK, GLA_ERR_INVALID_ARG, GLA_ERR_UNSUPPORTED, GLA_ERR_HIP = 0, 1, 2, 3
GLA_F32, GLA_BF16 = 0, 1
GLA_FWD, GLA_BWD = 0, 1

_lib = None
_lock = threading.Lock()


class GLAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load_library(path: str = LIB_PATH):
    """Open libgla.so and declare the C signatures.  Raises if the library is not built."""
    global _lib
    with _lock:
        if _lib is not None and path == LIB_PATH:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError("libgla.so is not built (%s); run `python -m sequence_state_scan_amd.build`" % path)
        lib = ctypes.CDLL(path)
        vp, fp, i = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
        lib.gla_supported.argtypes = [i, i, i, i]
        lib.gla_supported.restype = i
        lib.gla_status_string.argtypes = [i]
        lib.gla_status_string.restype = ctypes.c_char_p
        lib.gla_last_error.argtypes = []
        lib.gla_last_error.restype = ctypes.c_char_p
        lib.gla_chunk_fwd.argtypes = [vp, vp, vp, fp, vp, vp, fp, fp] + [i] * 8 + [vp]
        lib.gla_chunk_fwd.restype = i
        lib.gla_segment_scan.argtypes = [fp, fp, fp, fp, fp] + [i] * 7 + [vp]
        lib.gla_segment_scan.restype = i
        lib.gla_segment_scan_allgather.argtypes = [fp, fp, fp, fp, fp] + [i] * 6 + [vp]
        lib.gla_segment_scan_allgather.restype = i
        lib.gla_segment_correct.argtypes = [i, vp, vp, vp, fp, fp, fp, vp, vp, vp, vp, fp] + [i] * 8 + [vp]
        lib.gla_segment_correct.restype = i
        lib.gla_chunk_bwd.argtypes = [vp, vp, vp, fp, vp, vp, fp, vp, vp, vp, fp, fp] + [i] * 8 + [vp]
        lib.gla_chunk_bwd.restype = i
        if path == LIB_PATH:
            _lib = lib
        return lib


def declared_functions(header: str = HEADER):
    """Names of the functions include/gla.h declares."""
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(gla_\w+)\s*\(", text, re.M)))


def supported(dtype: torch.dtype, dk: int, dv: int, chunk: int) -> bool:
    return bool(load_library().gla_supported(_dtype_code(dtype), dk, dv, chunk))


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return GLA_BF16
    if dt == torch.float32:
        return GLA_F32
    raise TypeError("q, k, v must be torch.bfloat16 or torch.float32, got %s" % dt)


def _check(status: int):
    if status != GLA_OK:
        lib = load_library()
        raise GLAError(status, "%s: %s" % (lib.gla_status_string(status).decode(), lib.gla_last_error().decode()))


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libgla works on device tensors only (got a %s tensor)" % t.device)
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _f32(t, name):
    if t is not None and t.dtype != torch.float32:
        raise TypeError("%s must be float32" % name)
    return _p(t)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dims(q, v):
    B, H, T, dk = q.shape
    return B, H, T, dk, v.shape[-1]


# ------------------------------------------------------------------------------------ C calls

def chunk_states_dense(cs):
    """View of chunk states in the tiled layout of include/gla.h as ordinary row-major [dk][dv]
    states (a copy; for inspection and tests, not used by any entry point)."""
    *lead, dk, dv = cs.shape
    L = len(lead)
    if (dv // 16) % 2 == 1:
        t = cs.reshape(*lead, dk // 16, dv // 16, 4, 16, 4)  # tile row, tile column, j / 4, c, j % 4
        return t.permute(*range(L), L, L + 3, L + 1, L + 2, L + 4).reshape(*lead, dk, dv)
    # tile row, pair of tile columns, j / 4 within the tile, c, tile of the pair, j % 4
    t = cs.reshape(*lead, dk // 16, dv // 32, 4, 16, 2, 4)
    return t.permute(*range(L), L, L + 3, L + 1, L + 4, L + 2, L + 5).reshape(*lead, dk, dv)


def gla_chunk_fwd(q, k, v, g, chunk: int, P: int, o=None, chunk_states=None, seg_state=None, seg_logdecay=None):
    """Local pass.  Returns (o_local, chunk_states [B,H,T/chunk,dk,dv] (local, q's dtype, each
    state in the tiled layout: chunk_states_dense gives the row-major view),
    seg_state [B,H,P,dk,dv], seg_logdecay [B,H,P,dk])."""
    B, H, T, dk, dv = _dims(q, v)
    o = torch.empty_like(v) if o is None else o
    if chunk_states is None:
        chunk_states = torch.empty((B, H, T // chunk, dk, dv), device=q.device, dtype=q.dtype)
    if seg_state is None:
        seg_state = torch.empty((B, H, P, dk, dv), device=q.device, dtype=torch.float32)
    if seg_logdecay is None:
        seg_logdecay = torch.empty((B, H, P, dk), device=q.device, dtype=torch.float32)
    _check(load_library().gla_chunk_fwd(_p(q), _p(k), _p(v), _f32(g, "g"), _p(o), _p(chunk_states),
                                        _f32(seg_state, "seg_state"), _f32(seg_logdecay, "seg_logdecay"),
                                        B, H, T, dk, dv, chunk, P, _dtype_code(q.dtype), _stream(q)))
    return o, chunk_states, seg_state, seg_logdecay


def gla_segment_scan(seg_state, seg_logdecay, K: int, h_boundary=None, reverse: bool = False,
                     seg_carry=None, h_out=None, want_h_out: bool = True):
    """Decay-and-add scan over segments.  Returns (seg_carry, h_out)."""
    B, H, P, dk, dv = seg_state.shape
    seg_carry = torch.empty_like(seg_state) if seg_carry is None else seg_carry
    if h_out is None and want_h_out:
        h_out = torch.empty((B, H, dk, dv), device=seg_state.device, dtype=torch.float32)
    _check(load_library().gla_segment_scan(_f32(seg_state, "seg_state"), _f32(seg_logdecay, "seg_logdecay"),
                                           _f32(h_boundary, "h_boundary"), _f32(seg_carry, "seg_carry"),
                                           _f32(h_out, "h_out"), B, H, P, dk, dv, K, int(bool(reverse)),
                                           _stream(seg_state)))
    return seg_carry, h_out


def gla_segment_scan_allgather(seg_state, seg_logdecay, h_boundary=None, reverse: bool = False,
                               seg_carry=None, h_out=None, want_h_out: bool = True):
    """The same scan in the all-gather order (every carry combined directly from all the local
    states it depends on).  Returns (seg_carry, h_out)."""
    B, H, P, dk, dv = seg_state.shape
    seg_carry = torch.empty_like(seg_state) if seg_carry is None else seg_carry
    if h_out is None and want_h_out:
        h_out = torch.empty((B, H, dk, dv), device=seg_state.device, dtype=torch.float32)
    _check(load_library().gla_segment_scan_allgather(_f32(seg_state, "seg_state"), _f32(seg_logdecay, "seg_logdecay"),
                                                     _f32(h_boundary, "h_boundary"), _f32(seg_carry, "seg_carry"),
                                                     _f32(h_out, "h_out"), B, H, P, dk, dv, int(bool(reverse)),
                                                     _stream(seg_state)))
    return seg_carry, h_out


def _scan(method: str, seg_state, seg_logdecay, K: int, h_boundary, reverse: bool):
    if method == "chain":
        return gla_segment_scan(seg_state, seg_logdecay, K, h_boundary=h_boundary, reverse=reverse)
    if method == "allgather":
        return gla_segment_scan_allgather(seg_state, seg_logdecay, h_boundary=h_boundary, reverse=reverse)
    raise ValueError("unknown scan method %r" % method)


def gla_segment_correct(mode: int, chunk: int, P: int, q=None, k=None, v=None, g=None, seg_in=None,
                        seg_grad=None, o=None, chunk_states=None, dk=None, dv=None, dg=None):
    """Cumulative-decay correction, in place: o and chunk_states for GLA_FWD; dk, dv, dg for
    GLA_BWD (which reads the global chunk_states)."""
    ref_k = q if mode == GLA_FWD else k
    ref_v = o if mode == GLA_FWD else dv
    B, H, T, d_k = ref_k.shape
    d_v = ref_v.shape[-1]
    _check(load_library().gla_segment_correct(mode, _p(q), _p(k), _p(v), _f32(g, "g"), _f32(seg_in, "seg_in"),
                                              _f32(seg_grad, "seg_grad"), _p(o), _p(chunk_states), _p(dk), _p(dv),
                                              _f32(dg, "dg"), B, H, T, d_k, d_v, chunk, P,
                                              _dtype_code(ref_k.dtype), _stream(ref_k)))


def gla_chunk_bwd(q, k, v, g, do, chunk_states, seg_in, chunk: int, P: int, dq=None, dk=None, dv=None,
                  dg=None, seg_dstate=None):
    """Backward of every segment given the global chunk states and incoming segment states.

    Returns (dq global, dk local, dv local, dg local, seg_dstate [B,H,P,dk,dv])."""
    B, H, T, d_k, d_v = _dims(q, v)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dg = torch.empty_like(g) if dg is None else dg
    if seg_dstate is None:
        seg_dstate = torch.empty((B, H, P, d_k, d_v), device=q.device, dtype=torch.float32)
    _check(load_library().gla_chunk_bwd(_p(q), _p(k), _p(v), _f32(g, "g"), _p(do), _p(chunk_states),
                                        _f32(seg_in, "seg_in"), _p(dq), _p(dk), _p(dv), _f32(dg, "dg"),
                                        _f32(seg_dstate, "seg_dstate"), B, H, T, d_k, d_v, chunk, P,
                                        _dtype_code(q.dtype), _stream(q)))
    return dq, dk, dv, dg, seg_dstate


# ------------------------------------------------------------------------------ method chains

def zeco_forward(q, k, v, g, chunk: int, P: int, K: int, h0=None, scan: str = "chain"):
    """Local pass -> forward segment scan -> correction.  Returns a dict of tensors:
    o (global output), chunk_states (global state after every chunk), seg_in (state entering
    each segment), h_final (state after the last token), seg_state / seg_logdecay (local pass).
    scan: "chain" (gla_segment_scan) or "allgather" (gla_segment_scan_allgather)."""
    o, chunk_states, seg_state, seg_logdecay = gla_chunk_fwd(q, k, v, g, chunk, P)
    seg_in, h_final = _scan(scan, seg_state, seg_logdecay, K, h0, False)
    gla_segment_correct(GLA_FWD, chunk, P, q=q, g=g, seg_in=seg_in, o=o, chunk_states=chunk_states)
    return {"o": o, "chunk_states": chunk_states, "seg_in": seg_in, "h_final": h_final, "seg_state": seg_state,
            "seg_logdecay": seg_logdecay}


def zeco_backward(q, k, v, g, do, fwd: dict, chunk: int, P: int, K: int, dhT=None, scan: str = "chain"):
    """Local backward -> reverse segment scan -> gradient correction.  ``fwd`` is the dict
    zeco_forward returned.  Returns dq, dk, dv, dg, dh0 (and the intermediates)."""
    dq, dk, dv, dg, seg_dstate = gla_chunk_bwd(q, k, v, g, do, fwd["chunk_states"], fwd["seg_in"], chunk, P)
    seg_grad, dh0 = _scan(scan, seg_dstate, fwd["seg_logdecay"], K, dhT, True)
    gla_segment_correct(GLA_BWD, chunk, P, k=k, v=v, g=g, seg_in=fwd["seg_in"], seg_grad=seg_grad,
                        chunk_states=fwd["chunk_states"], dk=dk, dv=dv, dg=dg)
    return {"dq": dq, "dk": dk, "dv": dv, "dg": dg, "dh0": dh0, "seg_dstate": seg_dstate, "seg_grad": seg_grad}
