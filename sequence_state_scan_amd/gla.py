"""Thin ctypes binding of libgla.so (C ABI in include/gla.h).

Argument marshalling only: every step runs in the HIP kernels of libgla.so.  torch provides
device memory (tensors) and the stream (torch's current stream on the tensors' device).
There is no CPU fallback: without the built library every call raises.

Low-level calls carry the C names (gla_chunk_fwd, gla_segment_scan, gla_segment_correct,
gla_chunk_bwd, and for the other order gla_chunk_state, gla_chunk_fwd_from, gla_chunk_dstate,
gla_chunk_bwd_from).  ``zeco_forward`` / ``zeco_backward`` chain them in the order of the method:
local pass -> segment scan -> correction, and the same for the backward.
``states_first_forward`` / ``states_first_backward`` chain the same decomposition with the
segments' incoming states first: state pass -> segment scan -> local pass from the true incoming
state, with no correction pass (cheaper where the decay is weak and the corrections would reach
every chunk).
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
        sz = ctypes.c_size_t
        lib.gla_workspace_size.argtypes = [i] * 9
        lib.gla_workspace_size.restype = sz
        lib.gla_chunk_fwd.argtypes = [vp, vp, vp, fp, vp, vp, fp, fp] + [i] * 8 + [vp, sz, vp]
        lib.gla_chunk_fwd.restype = i
        lib.gla_chunk_fwd_noalloc.argtypes = [vp, vp, vp, fp, vp, vp, fp, fp] + [i] * 8 + [vp]
        lib.gla_chunk_fwd_noalloc.restype = i
        lib.gla_segment_scan.argtypes = [fp, fp, fp, fp, fp] + [i] * 7 + [vp]
        lib.gla_segment_scan.restype = i
        lib.gla_segment_scan_allgather.argtypes = [fp, fp, fp, fp, fp] + [i] * 6 + [vp]
        lib.gla_segment_scan_allgather.restype = i
        lib.gla_segment_correct.argtypes = [i, vp, vp, vp, fp, fp, fp, vp, vp, vp, vp, fp] + [i] * 8 + [vp]
        lib.gla_segment_correct.restype = i
        lib.gla_chunk_bwd.argtypes = [vp, vp, vp, fp, vp, vp, fp, vp, vp, vp, fp, fp] + [i] * 8 + [vp, sz, vp]
        lib.gla_chunk_bwd.restype = i
        lib.gla_chunk_state.argtypes = [vp, vp, fp, fp, fp] + [i] * 8 + [vp, sz, vp]
        lib.gla_chunk_state.restype = i
        lib.gla_chunk_fwd_from.argtypes = [vp, vp, vp, fp, fp, vp, vp] + [i] * 8 + [vp, sz, vp]
        lib.gla_chunk_fwd_from.restype = i
        lib.gla_chunk_dstate.argtypes = [vp, fp, vp, fp] + [i] * 8 + [vp, sz, vp]
        lib.gla_chunk_dstate.restype = i
        lib.gla_chunk_bwd_from.argtypes = [vp, vp, vp, fp, vp, vp, fp, fp, vp, vp, vp, fp] + [i] * 8 + [vp, sz, vp]
        lib.gla_chunk_bwd_from.restype = i
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


def _expect(t, name, shape, dtype, device, optional=False):
    """Check one tensor argument against the shape, dtype and device the call implies.  The
    kernels index every buffer from (B, H, T, dk, dv, P, chunk) alone, so a mismatch here would
    read or write outside the buffer: it is rejected before anything reaches the library."""
    if t is None:
        if optional:
            return
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dims(q, v):
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be [B, H, T, d] tensors")
    B, H, T, dk = q.shape
    return B, H, T, dk, v.shape[-1]


def _head_args(q, k, v, g, extra=()):
    """(B, H, T, dk, dv) from q and v, after checking q, k, v, g and the (name, tensor, last dim)
    triples of ``extra`` that share their [B, H, T] layout."""
    B, H, T, dk, dv = _dims(q, v)
    if not q.is_cuda:
        raise ValueError("libgla works on device tensors only (got a %s tensor)" % q.device)
    _dtype_code(q.dtype)
    _expect(q, "q", (B, H, T, dk), q.dtype, q.device)
    _expect(k, "k", (B, H, T, dk), q.dtype, q.device)
    _expect(v, "v", (B, H, T, dv), q.dtype, q.device)
    _expect(g, "g", (B, H, T, dk), torch.float32, q.device)
    for name, t, d, dt in extra:
        _expect(t, name, (B, H, T, d), dt, q.device)
    return B, H, T, dk, dv


def workspace_size(which: int, B: int, H: int, T: int, dk: int, dv: int, chunk: int, P: int, dtype) -> int:
    """Bytes of workspace gla_chunk_fwd (which=GLA_FWD) or gla_chunk_bwd (GLA_BWD) needs."""
    lib = load_library()
    n = lib.gla_workspace_size(which, B, H, T, dk, dv, chunk, P, _dtype_code(dtype))
    if n == 0:
        raise GLAError(GLA_ERR_INVALID_ARG, "gla_workspace_size: %s" % lib.gla_last_error().decode())
    return int(n)


def flags_workspace_size(B: int, H: int, P: int) -> int:
    """The smallest workspace gla_chunk_fwd / gla_chunk_bwd accept (include/gla.h,
    gla_workspace_size): one int per unit (b, h, segment), rounded up to 256 bytes.  With it a call
    cuts no segment into sub-segments and runs the units it flags whole (no re-split)."""
    return (B * H * P * 4 + 255) // 256 * 256


def _workspace(ws, which, B, H, T, dk, dv, chunk, P, dtype, device):
    """The caller's workspace, or one of the size for the fastest schedule.  A smaller one is the
    library's to accept (no re-split, fewer sub-segments) or reject, before any HIP call."""
    if ws is None:
        ws = torch.empty(workspace_size(which, B, H, T, dk, dv, chunk, P, dtype), dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % device)
    return ws, ws.numel() * ws.element_size()


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


def _seg_shapes(B, H, T, dk, dv, chunk, P):
    if P < 1 or chunk < 1 or T % P != 0 or (T // P) % chunk != 0:
        raise ValueError("T=%d must split into P=%d segments of whole chunks of %d tokens" % (T, P, chunk))
    return (B, H, T // chunk, dk, dv), (B, H, P, dk, dv), (B, H, P, dk)


def gla_chunk_fwd(q, k, v, g, chunk: int, P: int, o=None, chunk_states=None, seg_state=None, seg_logdecay=None,
                  workspace=None, keep_chunk_states: bool = True):
    """Local pass.  Returns (o_local, chunk_states [B,H,T/chunk,dk,dv] (local, q's dtype, each
    state in the tiled layout: chunk_states_dense gives the row-major view),
    seg_state [B,H,P,dk,dv], seg_logdecay [B,H,P,dk]).  ``workspace`` (a device tensor of at
    least workspace_size(GLA_FWD, ...) bytes) is allocated when not given.
    keep_chunk_states=False (a forward-only caller: no backward follows) keeps no per-chunk states
    and returns None in their place; the other results are the same bit for bit."""
    B, H, T, dk, dv = _head_args(q, k, v, g)
    cs_shape, st_shape, ld_shape = _seg_shapes(B, H, T, dk, dv, chunk, P)
    dev, f32 = q.device, torch.float32
    o = torch.empty_like(v) if o is None else o
    if not keep_chunk_states:
        if chunk_states is not None:
            raise ValueError("chunk_states given with keep_chunk_states=False")
    elif chunk_states is None:
        chunk_states = torch.empty(cs_shape, device=dev, dtype=q.dtype)
    if seg_state is None:
        seg_state = torch.empty(st_shape, device=dev, dtype=f32)
    if seg_logdecay is None:
        seg_logdecay = torch.empty(ld_shape, device=dev, dtype=f32)
    _expect(o, "o", (B, H, T, dv), q.dtype, dev)
    _expect(chunk_states, "chunk_states", cs_shape, q.dtype, dev, optional=not keep_chunk_states)
    _expect(seg_state, "seg_state", st_shape, f32, dev)
    _expect(seg_logdecay, "seg_logdecay", ld_shape, f32, dev)
    ws, nbytes = _workspace(workspace, GLA_FWD, B, H, T, dk, dv, chunk, P, q.dtype, dev)
    _check(load_library().gla_chunk_fwd(_p(q), _p(k), _p(v), _p(g), _p(o), _p(chunk_states), _p(seg_state),
                                        _p(seg_logdecay), B, H, T, dk, dv, chunk, P, _dtype_code(q.dtype),
                                        _p(ws), nbytes, _stream(q)))
    return o, chunk_states, seg_state, seg_logdecay


def gla_chunk_fwd_noalloc(q, k, v, g, chunk: int, P: int, o, chunk_states, seg_state, seg_logdecay):
    """gla_chunk_fwd without a workspace (the library's static one): every output is the caller's
    and must be given (chunk_states may be None: no per-chunk states kept); nothing is allocated."""
    B, H, T, dk, dv = _head_args(q, k, v, g)
    cs_shape, st_shape, ld_shape = _seg_shapes(B, H, T, dk, dv, chunk, P)
    dev, f32 = q.device, torch.float32
    _expect(o, "o", (B, H, T, dv), q.dtype, dev)
    _expect(chunk_states, "chunk_states", cs_shape, q.dtype, dev, optional=True)
    _expect(seg_state, "seg_state", st_shape, f32, dev)
    _expect(seg_logdecay, "seg_logdecay", ld_shape, f32, dev)
    _check(load_library().gla_chunk_fwd_noalloc(_p(q), _p(k), _p(v), _p(g), _p(o), _p(chunk_states), _p(seg_state),
                                                _p(seg_logdecay), B, H, T, dk, dv, chunk, P, _dtype_code(q.dtype),
                                                _stream(q)))
    return o, chunk_states, seg_state, seg_logdecay


def _scan_args(seg_state, seg_logdecay, h_boundary, seg_carry, h_out, want_h_out):
    if not isinstance(seg_state, torch.Tensor) or seg_state.dim() != 5:
        raise ValueError("seg_state must be a [B, H, P, dk, dv] tensor")
    B, H, P, dk, dv = seg_state.shape
    dev, f32 = seg_state.device, torch.float32
    _expect(seg_state, "seg_state", (B, H, P, dk, dv), f32, dev)
    _expect(seg_logdecay, "seg_logdecay", (B, H, P, dk), f32, dev)
    _expect(h_boundary, "h_boundary", (B, H, dk, dv), f32, dev, optional=True)
    seg_carry = torch.empty_like(seg_state) if seg_carry is None else seg_carry
    _expect(seg_carry, "seg_carry", (B, H, P, dk, dv), f32, dev)
    if h_out is None and want_h_out:
        h_out = torch.empty((B, H, dk, dv), device=dev, dtype=f32)
    _expect(h_out, "h_out", (B, H, dk, dv), f32, dev, optional=True)
    return B, H, P, dk, dv, seg_carry, h_out


def gla_segment_scan(seg_state, seg_logdecay, K: int, h_boundary=None, reverse: bool = False,
                     seg_carry=None, h_out=None, want_h_out: bool = True):
    """Decay-and-add scan over segments.  Returns (seg_carry, h_out)."""
    B, H, P, dk, dv, seg_carry, h_out = _scan_args(seg_state, seg_logdecay, h_boundary, seg_carry, h_out, want_h_out)
    _check(load_library().gla_segment_scan(_f32(seg_state, "seg_state"), _f32(seg_logdecay, "seg_logdecay"),
                                           _f32(h_boundary, "h_boundary"), _f32(seg_carry, "seg_carry"),
                                           _f32(h_out, "h_out"), B, H, P, dk, dv, K, int(bool(reverse)),
                                           _stream(seg_state)))
    return seg_carry, h_out


def gla_segment_scan_allgather(seg_state, seg_logdecay, h_boundary=None, reverse: bool = False,
                               seg_carry=None, h_out=None, want_h_out: bool = True):
    """The same scan in the all-gather order (every carry combined directly from all the local
    states it depends on).  Returns (seg_carry, h_out)."""
    B, H, P, dk, dv, seg_carry, h_out = _scan_args(seg_state, seg_logdecay, h_boundary, seg_carry, h_out, want_h_out)
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
    if mode not in (GLA_FWD, GLA_BWD):
        raise ValueError("mode must be GLA_FWD or GLA_BWD")
    ref_k = q if mode == GLA_FWD else k
    ref_v = o if mode == GLA_FWD else dv
    if ref_k is None or ref_v is None:
        raise ValueError("GLA_FWD needs q and o, GLA_BWD needs k and dv")
    B, H, T, d_k, d_v = _dims(ref_k, ref_v)
    dt, dev, f32 = ref_k.dtype, ref_k.device, torch.float32
    cs_shape, st_shape, _ = _seg_shapes(B, H, T, d_k, d_v, chunk, P)
    _expect(g, "g", (B, H, T, d_k), f32, dev)
    _expect(seg_in, "seg_in", st_shape, f32, dev)
    # GLA_FWD may go without chunk states (a forward-only caller kept none)
    _expect(chunk_states, "chunk_states", cs_shape, dt, dev, optional=mode == GLA_FWD)
    if mode == GLA_FWD:
        _expect(q, "q", (B, H, T, d_k), dt, dev)
        _expect(o, "o", (B, H, T, d_v), dt, dev)
    else:
        for name, t, d in (("k", k, d_k), ("v", v, d_v), ("dk", dk, d_k), ("dv", dv, d_v)):
            _expect(t, name, (B, H, T, d), dt, dev)
        _expect(dg, "dg", (B, H, T, d_k), f32, dev)
        _expect(seg_grad, "seg_grad", st_shape, f32, dev)
    _check(load_library().gla_segment_correct(mode, _p(q), _p(k), _p(v), _f32(g, "g"), _f32(seg_in, "seg_in"),
                                              _f32(seg_grad, "seg_grad"), _p(o), _p(chunk_states), _p(dk), _p(dv),
                                              _f32(dg, "dg"), B, H, T, d_k, d_v, chunk, P,
                                              _dtype_code(ref_k.dtype), _stream(ref_k)))


def gla_chunk_bwd(q, k, v, g, do, chunk_states, seg_in, chunk: int, P: int, dq=None, dk=None, dv=None,
                  dg=None, seg_dstate=None, workspace=None):
    """Backward of every segment given the global chunk states and incoming segment states.

    Returns (dq global, dk local, dv local, dg local, seg_dstate [B,H,P,dk,dv]).  ``workspace`` as
    in gla_chunk_fwd (GLA_BWD size)."""
    B, H, T, d_k, d_v = _head_args(q, k, v, g, (("do", do, v.shape[-1], q.dtype),))
    cs_shape, st_shape, _ = _seg_shapes(B, H, T, d_k, d_v, chunk, P)
    dev, f32 = q.device, torch.float32
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dg = torch.empty_like(g) if dg is None else dg
    if seg_dstate is None:
        seg_dstate = torch.empty(st_shape, device=dev, dtype=f32)
    _expect(chunk_states, "chunk_states", cs_shape, q.dtype, dev)
    _expect(seg_in, "seg_in", st_shape, f32, dev)
    for name, t, d in (("dq", dq, d_k), ("dk", dk, d_k), ("dv", dv, d_v)):
        _expect(t, name, (B, H, T, d), q.dtype, dev)
    _expect(dg, "dg", (B, H, T, d_k), f32, dev)
    _expect(seg_dstate, "seg_dstate", st_shape, f32, dev)
    ws, nbytes = _workspace(workspace, GLA_BWD, B, H, T, d_k, d_v, chunk, P, q.dtype, dev)
    _check(load_library().gla_chunk_bwd(_p(q), _p(k), _p(v), _p(g), _p(do), _p(chunk_states), _p(seg_in),
                                        _p(dq), _p(dk), _p(dv), _p(dg), _p(seg_dstate), B, H, T, d_k, d_v, chunk,
                                        P, _dtype_code(q.dtype), _p(ws), nbytes, _stream(q)))
    return dq, dk, dv, dg, seg_dstate


def _seg_args(name_a, a, v, g, extra=()):
    """(B, H, T, dk, dv) for the state passes, whose inputs are a ([B,H,T,dk]: k or q), v or do
    ([B,H,T,dv]) and g, after checking them and ``extra``'s (name, tensor, last dim, dtype)."""
    if not isinstance(a, torch.Tensor) or not isinstance(v, torch.Tensor) or a.dim() != 4 or v.dim() != 4:
        raise ValueError("%s and the value-side input must be [B, H, T, d] tensors" % name_a)
    B, H, T, dk = a.shape
    dv = v.shape[-1]
    if not a.is_cuda:
        raise ValueError("libgla works on device tensors only (got a %s tensor)" % a.device)
    _dtype_code(a.dtype)
    _expect(a, name_a, (B, H, T, dk), a.dtype, a.device)
    _expect(g, "g", (B, H, T, dk), torch.float32, a.device)
    for name, t, d, dt in extra:
        _expect(t, name, (B, H, T, d), dt, a.device)
    return B, H, T, dk, dv


def gla_chunk_state(k, v, g, chunk: int, P: int, seg_state=None, seg_logdecay=None, workspace=None):
    """State pass: each segment's local end state and summed log-gates from a zero start (reads k,
    v, g only).  Returns (seg_state [B,H,P,dk,dv], seg_logdecay [B,H,P,dk]), the same quantities as
    gla_chunk_fwd's.  ``workspace`` (GLA_FWD size) lets it cut segments into sub-segments."""
    B, H, T, dk, dv = _seg_args("k", k, v, g, (("v", v, v.shape[-1], k.dtype),))
    _, st_shape, ld_shape = _seg_shapes(B, H, T, dk, dv, chunk, P)
    dev, f32 = k.device, torch.float32
    seg_state = torch.empty(st_shape, device=dev, dtype=f32) if seg_state is None else seg_state
    seg_logdecay = torch.empty(ld_shape, device=dev, dtype=f32) if seg_logdecay is None else seg_logdecay
    _expect(seg_state, "seg_state", st_shape, f32, dev)
    _expect(seg_logdecay, "seg_logdecay", ld_shape, f32, dev)
    ws, nbytes = _workspace(workspace, GLA_FWD, B, H, T, dk, dv, chunk, P, k.dtype, dev)
    _check(load_library().gla_chunk_state(_p(k), _p(v), _p(g), _p(seg_state), _p(seg_logdecay), B, H, T, dk, dv,
                                          chunk, P, _dtype_code(k.dtype), _p(ws), nbytes, _stream(k)))
    return seg_state, seg_logdecay


def gla_chunk_fwd_from(q, k, v, g, seg_in, chunk: int, P: int, o=None, chunk_states=None, workspace=None,
                       keep_chunk_states: bool = True):
    """Local pass with every segment starting from its true incoming state seg_in [B,H,P,dk,dv]
    (the forward scan's carry): returns (o, chunk_states), both GLOBAL; no correction follows.
    chunk_states (tiled layout) is None with keep_chunk_states=False."""
    B, H, T, dk, dv = _head_args(q, k, v, g)
    cs_shape, st_shape, _ = _seg_shapes(B, H, T, dk, dv, chunk, P)
    dev = q.device
    o = torch.empty_like(v) if o is None else o
    if not keep_chunk_states:
        if chunk_states is not None:
            raise ValueError("chunk_states given with keep_chunk_states=False")
    elif chunk_states is None:
        chunk_states = torch.empty(cs_shape, device=dev, dtype=q.dtype)
    _expect(seg_in, "seg_in", st_shape, torch.float32, dev)
    _expect(o, "o", (B, H, T, dv), q.dtype, dev)
    _expect(chunk_states, "chunk_states", cs_shape, q.dtype, dev, optional=not keep_chunk_states)
    ws, nbytes = _workspace(workspace, GLA_FWD, B, H, T, dk, dv, chunk, P, q.dtype, dev)
    _check(load_library().gla_chunk_fwd_from(_p(q), _p(k), _p(v), _p(g), _p(seg_in), _p(o), _p(chunk_states), B, H,
                                             T, dk, dv, chunk, P, _dtype_code(q.dtype), _p(ws), nbytes, _stream(q)))
    return o, chunk_states


def gla_chunk_dstate(q, g, do, chunk: int, P: int, seg_dstate=None, workspace=None):
    """State-gradient pass: each segment's gradient w.r.t. its incoming state from its own outputs
    (reads q, g, do only).  Returns seg_dstate [B,H,P,dk,dv], the same quantity as gla_chunk_bwd's.
    ``workspace`` (GLA_BWD size) lets it cut segments into sub-segments."""
    B, H, T, dk, dv = _seg_args("q", q, do, g, (("do", do, do.shape[-1], q.dtype),))
    _, st_shape, _ = _seg_shapes(B, H, T, dk, dv, chunk, P)
    dev = q.device
    seg_dstate = torch.empty(st_shape, device=dev, dtype=torch.float32) if seg_dstate is None else seg_dstate
    _expect(seg_dstate, "seg_dstate", st_shape, torch.float32, dev)
    ws, nbytes = _workspace(workspace, GLA_BWD, B, H, T, dk, dv, chunk, P, q.dtype, dev)
    _check(load_library().gla_chunk_dstate(_p(q), _p(g), _p(do), _p(seg_dstate), B, H, T, dk, dv, chunk, P,
                                           _dtype_code(q.dtype), _p(ws), nbytes, _stream(q)))
    return seg_dstate


def gla_chunk_bwd_from(q, k, v, g, do, chunk_states, seg_in, seg_grad, chunk: int, P: int, dq=None, dk=None,
                       dv=None, dg=None, workspace=None):
    """Backward of every segment starting from seg_grad [B,H,P,dk,dv] (the reverse scan's carry)
    at its end, given the global chunk states and incoming states: returns (dq, dk, dv, dg), all
    GLOBAL; no correction follows."""
    B, H, T, d_k, d_v = _head_args(q, k, v, g, (("do", do, v.shape[-1], q.dtype),))
    cs_shape, st_shape, _ = _seg_shapes(B, H, T, d_k, d_v, chunk, P)
    dev, f32 = q.device, torch.float32
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dg = torch.empty_like(g) if dg is None else dg
    _expect(chunk_states, "chunk_states", cs_shape, q.dtype, dev)
    _expect(seg_in, "seg_in", st_shape, f32, dev)
    _expect(seg_grad, "seg_grad", st_shape, f32, dev)
    for name, t, d in (("dq", dq, d_k), ("dk", dk, d_k), ("dv", dv, d_v)):
        _expect(t, name, (B, H, T, d), q.dtype, dev)
    _expect(dg, "dg", (B, H, T, d_k), f32, dev)
    ws, nbytes = _workspace(workspace, GLA_BWD, B, H, T, d_k, d_v, chunk, P, q.dtype, dev)
    _check(load_library().gla_chunk_bwd_from(_p(q), _p(k), _p(v), _p(g), _p(do), _p(chunk_states), _p(seg_in),
                                             _p(seg_grad), _p(dq), _p(dk), _p(dv), _p(dg), B, H, T, d_k, d_v, chunk,
                                             P, _dtype_code(q.dtype), _p(ws), nbytes, _stream(q)))
    return dq, dk, dv, dg


# ------------------------------------------------------------------------------ method chains

def zeco_forward(q, k, v, g, chunk: int, P: int, K: int, h0=None, scan: str = "chain",
                 keep_chunk_states: bool = True):
    """Local pass -> forward segment scan -> correction.  Returns a dict of tensors:
    o (global output), chunk_states (global state after every chunk; None with
    keep_chunk_states=False, for a forward-only caller), seg_in (state entering each segment),
    h_final (state after the last token), seg_state / seg_logdecay (local pass).
    scan: "chain" (gla_segment_scan) or "allgather" (gla_segment_scan_allgather)."""
    o, chunk_states, seg_state, seg_logdecay = gla_chunk_fwd(q, k, v, g, chunk, P,
                                                             keep_chunk_states=keep_chunk_states)
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


def states_first_segments(B: int, H: int, T: int, chunk: int, P: int) -> int:
    """The segment count the order with the incoming states first runs at: P, each segment cut in
    two while the B*H*P' units leave CUs idle (fewer than 256) and the halves keep at least 2
    chunks.  In this order nothing depends on the segmentation beyond rounding (there is no
    correction whose work grows with it), and with P' segments no call cuts sub-segments of its
    own, whose state pass would repeat gla_chunk_state's."""
    if P < 1 or chunk < 1 or T % P or (T // P) % chunk:
        raise ValueError("T=%d must split into P=%d segments of whole chunks of %d tokens" % (T, P, chunk))
    n = T // P // chunk
    while B * H * P < 256 and n % 2 == 0 and n // 2 >= 2:
        P, n = 2 * P, n // 2
    return P


def states_first_forward(q, k, v, g, chunk: int, P: int, K: int, h0=None, scan: str = "chain",
                         keep_chunk_states: bool = True, fill: bool = True):
    """The same forward with the incoming states first: state pass -> forward segment scan ->
    local pass from each segment's true incoming state (no correction).  With fill, the segments
    are first cut to fill the chip (states_first_segments); the per-segment results then count
    those segments, whose number the dict holds as "P".  Returns the dict zeco_forward returns
    (o, chunk_states, seg_in, h_final, seg_state, seg_logdecay) plus "P"."""
    if fill:
        P = states_first_segments(q.shape[0], q.shape[1], q.shape[2], chunk, P)
    seg_state, seg_logdecay = gla_chunk_state(k, v, g, chunk, P)
    seg_in, h_final = _scan(scan, seg_state, seg_logdecay, K, h0, False)
    o, chunk_states = gla_chunk_fwd_from(q, k, v, g, seg_in, chunk, P, keep_chunk_states=keep_chunk_states)
    return {"o": o, "chunk_states": chunk_states, "seg_in": seg_in, "h_final": h_final, "seg_state": seg_state,
            "seg_logdecay": seg_logdecay, "P": P}


def states_first_backward(q, k, v, g, do, fwd: dict, chunk: int, K: int, dhT=None, scan: str = "chain"):
    """The same backward with the incoming gradients first: state-gradient pass -> reverse segment
    scan -> local backward from each segment's true outgoing gradient (no correction), over the
    segments of ``fwd``, the dict states_first_forward returned.  Returns the dict zeco_backward
    returns."""
    P = fwd["P"]
    seg_dstate = gla_chunk_dstate(q, g, do, chunk, P)
    seg_grad, dh0 = _scan(scan, seg_dstate, fwd["seg_logdecay"], K, dhT, True)
    dq, dk, dv, dg = gla_chunk_bwd_from(q, k, v, g, do, fwd["chunk_states"], fwd["seg_in"], seg_grad, chunk, P)
    return {"dq": dq, "dk": dk, "dv": dv, "dg": dg, "dh0": dh0, "seg_dstate": seg_dstate, "seg_grad": seg_grad}


# ------------------------------------------------------------------------ several streams at once

_streams = {}


def _side_streams(device, n):
    """n streams of default priority on ``device``, created once and reused."""
    key = (device.index, n)
    if key not in _streams:
        _streams[key] = [torch.cuda.Stream(device=device) for _ in range(n)]
    return _streams[key]


def _rows(t, lo, hi):
    """Sequences lo..hi-1 of a [B, H, ...] tensor, as a contiguous [hi-lo, 1, ...] view."""
    if t is None:
        return None
    flat = t.view(t.shape[0] * t.shape[1], 1, *t.shape[2:])
    return flat[lo:hi]


def zeco_step_streams(q, k, v, g, do, chunk: int, P: int, K: int, n_streams: int = 2, h0=None, dhT=None,
                      out=None, stagger: bool = False):
    """The whole fwd+bwd path with the B*H sequences cut into ``n_streams`` groups, each group's six
    calls (local pass, scan, correction; local backward, reverse scan, correction) in order on a
    stream of its own.  The streams fork from torch's current stream and join back into it, so
    the result is ordered like any other call on the current stream.  While one group runs its
    scans and corrections, another group's local passes can use the CUs they leave free.  The
    groups' calls get flag-only workspaces, so none cuts its segments into sub-segments: every unit
    is computed exactly as in the one-stream chain run with such workspaces, bit for bit.

    ``out``: optional dict of preallocated buffers (as returned by a previous call) to reuse.
    ``stagger``: each group's chain waits for the previous group's local pass, so that a group's
    scan and correction run while the next group's local pass does (the overlap the ZeCO pages
    measure; on one GPU it serialises the local passes of the groups, which costs more than the
    scans it hides).
    Returns a dict: o, h_final, dq, dk, dv, dg, dh0 and the intermediates."""
    B, H, T, dk_, dv_ = _head_args(q, k, v, g, (("do", do, v.shape[-1], q.dtype),))
    cs_shape, st_shape, ld_shape = _seg_shapes(B, H, T, dk_, dv_, chunk, P)
    dev, f32, edt = q.device, torch.float32, q.dtype
    if out is None:
        out = {
            "o": torch.empty_like(v), "chunk_states": torch.empty(cs_shape, device=dev, dtype=edt),
            "seg_state": torch.empty(st_shape, device=dev, dtype=f32),
            "seg_logdecay": torch.empty(ld_shape, device=dev, dtype=f32),
            "seg_in": torch.empty(st_shape, device=dev, dtype=f32),
            "h_final": torch.empty((B, H, dk_, dv_), device=dev, dtype=f32),
            "dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
            "dg": torch.empty_like(g), "seg_dstate": torch.empty(st_shape, device=dev, dtype=f32),
            "seg_grad": torch.empty(st_shape, device=dev, dtype=f32),
            "dh0": torch.empty((B, H, dk_, dv_), device=dev, dtype=f32),
        }
    BH = B * H
    n = max(1, min(n_streams, BH))
    bounds = [BH * i // n for i in range(n + 1)]
    if "workspaces" not in out or len(out["workspaces"]) != n:
        # flags only: a group's calls cut no segment into sub-segments, because the groups share the
        # chip; each call on its own would cut its fewer units to fill it
        out["workspaces"] = [torch.empty(flags_workspace_size(bounds[i + 1] - bounds[i], 1, P), device=dev,
                                         dtype=torch.uint8) for i in range(n)]
    main = torch.cuda.current_stream(dev)
    streams = _side_streams(dev, n)
    local_done = None
    for i, st in enumerate(streams):
        lo, hi = bounds[i], bounds[i + 1]
        r = {name: _rows(t, lo, hi) for name, t in out.items() if isinstance(t, torch.Tensor)}
        x = {name: _rows(t, lo, hi) for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("do", do),
                                                     ("h0", h0), ("dhT", dhT))}
        ws = out["workspaces"][i]
        st.wait_stream(main)
        if stagger and local_done is not None:
            st.wait_event(local_done)
        with torch.cuda.stream(st):
            gla_chunk_fwd(x["q"], x["k"], x["v"], x["g"], chunk, P, o=r["o"], chunk_states=r["chunk_states"],
                          seg_state=r["seg_state"], seg_logdecay=r["seg_logdecay"], workspace=ws)
            if stagger:
                local_done = torch.cuda.Event()
                local_done.record(st)
            gla_segment_scan(r["seg_state"], r["seg_logdecay"], K, h_boundary=x["h0"], seg_carry=r["seg_in"],
                             h_out=r["h_final"])
            gla_segment_correct(GLA_FWD, chunk, P, q=x["q"], g=x["g"], seg_in=r["seg_in"], o=r["o"],
                                chunk_states=r["chunk_states"])
            gla_chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["do"], r["chunk_states"], r["seg_in"], chunk, P,
                          dq=r["dq"], dk=r["dk"], dv=r["dv"], dg=r["dg"], seg_dstate=r["seg_dstate"], workspace=ws)
            gla_segment_scan(r["seg_dstate"], r["seg_logdecay"], K, h_boundary=x["dhT"], reverse=True,
                             seg_carry=r["seg_grad"], h_out=r["dh0"])
            gla_segment_correct(GLA_BWD, chunk, P, k=x["k"], v=x["v"], g=x["g"], seg_in=r["seg_in"],
                                seg_grad=r["seg_grad"], chunk_states=r["chunk_states"], dk=r["dk"], dv=r["dv"],
                                dg=r["dg"])
    for st in streams:
        main.wait_stream(st)
    return out

