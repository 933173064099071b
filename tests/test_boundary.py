"""The C ABI without a GPU: libgla.so loads, exports every function include/gla.h declares, and
rejects bad arguments on the host before any HIP call (so these tests never launch anything).
"""
import ctypes

import pytest
import torch

from sequence_state_scan_amd import gla

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host checks
NUL = None


@pytest.fixture(scope="module")
def lib():
    return gla.load_library()


def test_every_declared_function_is_exported(lib):
    names = gla.declared_functions()
    assert {"gla_chunk_fwd", "gla_chunk_bwd", "gla_segment_scan", "gla_segment_correct"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.gla_status_string(0) == b"GLA_OK"
    assert lib.gla_status_string(1) == b"GLA_ERR_INVALID_ARG"
    assert lib.gla_status_string(2) == b"GLA_ERR_UNSUPPORTED"
    assert lib.gla_status_string(3) == b"GLA_ERR_HIP"


def test_supported_shape_table(lib):
    for dk, dv, c in [(128, 256, 64), (128, 128, 64), (64, 64, 32), (32, 32, 32), (128, 256, 32), (128, 256, 16),
                      (32, 32, 16)]:
        assert lib.gla_supported(gla.GLA_BF16, dk, dv, c) == 1, (dk, dv, c)
    for dk, dv, c in [(16, 16, 16), (32, 32, 64), (16, 32, 32)]:
        assert lib.gla_supported(gla.GLA_F32, dk, dv, c) == 1, (dk, dv, c)
    for dt, dk, dv, c in [(gla.GLA_BF16, 48, 64, 64), (gla.GLA_BF16, 128, 256, 8), (gla.GLA_BF16, 256, 256, 64),
                          (gla.GLA_F32, 128, 128, 64), (gla.GLA_F32, 16, 16, 8), (7, 64, 64, 64)]:
        assert lib.gla_supported(dt, dk, dv, c) == 0, (dt, dk, dv, c)


WS = ctypes.c_void_p(0xA000)  # a stand-in workspace pointer


def _fwd(lib, B=1, H=1, T=256, dk=64, dv=64, chunk=64, P=1, dtype=gla.GLA_BF16, q=FAKE, o=ctypes.c_void_p(0x2000),
         ss=FAKE, ws=WS, wsb=1 << 20):
    return lib.gla_chunk_fwd(q, FAKE, FAKE, FAKE, o, ctypes.c_void_p(0x4000), ss, FAKE, B, H, T, dk, dv, chunk, P,
                             dtype, ws, wsb, NUL)


def test_chunk_fwd_host_checks(lib):
    E, U = gla.GLA_ERR_INVALID_ARG, gla.GLA_ERR_UNSUPPORTED
    assert _fwd(lib, T=250, P=4) == E          # T % P != 0
    assert _fwd(lib, T=256, P=8) == E          # segment 32 not a multiple of chunk 64
    assert _fwd(lib, B=0) == E
    assert _fwd(lib, T=0) == E                 # empty sequence
    assert _fwd(lib, dtype=9) == E
    assert _fwd(lib, q=NUL) == E               # null input
    assert _fwd(lib, ss=NUL) == E              # null output
    assert _fwd(lib, o=FAKE) == E              # o aliases q
    assert _fwd(lib, dk=48) == U               # valid but no kernel built
    assert _fwd(lib, dk=256) == U              # d_k above 128 has no kernel
    assert _fwd(lib, chunk=8) == U             # no 8-token chunks
    assert _fwd(lib, ws=NUL) == E              # the workspace is required
    assert _fwd(lib, wsb=255) == E             # and must hold gla_workspace_size bytes
    assert b"workspace" in lib.gla_last_error()
    assert _fwd(lib, B=4, H=16, T=256 * 16, P=16, wsb=1023) == E  # 1024 bytes needed for 1024 units
    # a small problem is cut into sub-segments, so the fastest schedule needs more than the flags;
    # any size from the flags up is accepted (fewer sub-segments; run on the GPU by
    # test_small_workspace_runs_fewer_sub_segments)
    assert lib.gla_workspace_size(gla.GLA_FWD, 1, 1, 256, 64, 64, 64, 1, gla.GLA_BF16) > 256
    assert gla.flags_workspace_size(4, 16, 16) == 4096 and gla.flags_workspace_size(1, 1, 1) == 256
    assert _fwd(lib, ws=FAKE) == E             # the workspace aliases q


def test_segment_scan_host_checks(lib):
    E = gla.GLA_ERR_INVALID_ARG
    other = ctypes.c_void_p(0x3000)
    args = lambda K=2, rev=0, carry=other, st=FAKE: (st, FAKE, NUL, carry, NUL, 1, 1, 4, 16, 16, K, rev, NUL)  # noqa
    assert lib.gla_segment_scan(*args(K=3)) == E      # K does not divide dk
    assert lib.gla_segment_scan(*args(K=0)) == E
    assert lib.gla_segment_scan(*args(K=32)) == E     # K > dk
    assert lib.gla_segment_scan(*args(rev=2)) == E
    assert lib.gla_segment_scan(*args(carry=NUL)) == E
    assert lib.gla_segment_scan(*args(carry=FAKE)) == E  # carry aliases state


def test_segment_scan_allgather_host_checks(lib):
    E = gla.GLA_ERR_INVALID_ARG
    other = ctypes.c_void_p(0x3000)
    args = lambda rev=0, carry=other, P=4: (FAKE, FAKE, NUL, carry, NUL, 1, 1, P, 16, 16, rev, NUL)  # noqa
    assert lib.gla_segment_scan_allgather(*args(rev=2)) == E
    assert lib.gla_segment_scan_allgather(*args(P=0)) == E
    assert lib.gla_segment_scan_allgather(*args(carry=NUL)) == E
    assert lib.gla_segment_scan_allgather(*args(carry=FAKE)) == E  # carry aliases state


def test_segment_correct_host_checks(lib):
    E = gla.GLA_ERR_INVALID_ARG
    def call(mode, q=FAKE, k=FAKE, o=FAKE, dk=FAKE, T=256, P=4):
        return lib.gla_segment_correct(mode, q, k, FAKE, FAKE, FAKE, FAKE, o, FAKE, dk, FAKE, FAKE,
                                       1, 1, T, 32, 32, 32, P, gla.GLA_BF16, NUL)
    assert call(5) == E
    assert call(gla.GLA_FWD, q=NUL) == E
    assert call(gla.GLA_FWD, o=NUL) == E
    assert call(gla.GLA_BWD, k=NUL) == E
    assert call(gla.GLA_BWD, dk=NUL) == E
    assert call(gla.GLA_FWD, T=100, P=4) == E
    assert call(gla.GLA_BWD, T=0) == E         # empty sequence


def test_chunk_bwd_host_checks(lib):
    E = gla.GLA_ERR_INVALID_ARG
    def call(dq=ctypes.c_void_p(0x5000), dg=ctypes.c_void_p(0x6000), P=2, T=256):
        return lib.gla_chunk_bwd(FAKE, ctypes.c_void_p(0x1100), ctypes.c_void_p(0x1200), ctypes.c_void_p(0x1300),
                                 ctypes.c_void_p(0x1400), ctypes.c_void_p(0x1480), ctypes.c_void_p(0x1500), dq,
                                 ctypes.c_void_p(0x7000),
                                 ctypes.c_void_p(0x8000), dg, ctypes.c_void_p(0x9000),
                                 1, 1, T, 64, 64, 64, P, gla.GLA_BF16, WS, 256, NUL)
    assert call(dq=FAKE) == E      # dq aliases q
    assert call(dg=NUL) == E
    assert call(P=3) == E
    assert call(T=0) == E          # empty sequence
    ws_call = lambda ws, n: lib.gla_chunk_bwd(FAKE, ctypes.c_void_p(0x1100), ctypes.c_void_p(0x1200),  # noqa
                                              ctypes.c_void_p(0x1300), ctypes.c_void_p(0x1400),
                                              ctypes.c_void_p(0x1480), ctypes.c_void_p(0x1500),
                                              ctypes.c_void_p(0x5000), ctypes.c_void_p(0x7000),
                                              ctypes.c_void_p(0x8000), ctypes.c_void_p(0x6000),
                                              ctypes.c_void_p(0x9000), 1, 1, 256, 64, 64, 64, 2, gla.GLA_BF16,
                                              ws, n, NUL)
    assert ws_call(NUL, 256) == E
    assert ws_call(WS, 8) == E
    assert ws_call(ctypes.c_void_p(0x1480), 256) == E  # the workspace aliases chunk_states


def test_states_first_calls_host_checks(lib):
    # the calls of the order with the incoming states first reject bad arguments the same way
    E, U = gla.GLA_ERR_INVALID_ARG, gla.GLA_ERR_UNSUPPORTED
    A = [ctypes.c_void_p(0x1000 + 0x100 * i) for i in range(16)]  # distinct stand-in pointers

    def state(k=A[1], st=A[5], ld=A[6], T=256, P=2, chunk=64, dk=64, dtype=gla.GLA_BF16, ws=NUL, wsb=0):
        return lib.gla_chunk_state(k, A[2], A[3], st, ld, 1, 1, T, dk, 64, chunk, P, dtype, ws, wsb, NUL)

    assert state(k=NUL) == E
    assert state(st=NUL) == E
    assert state(ld=NUL) == E
    assert state(st=A[1]) == E                 # the output aliases k
    assert state(T=250) == E
    assert state(T=0) == E
    assert state(dk=48) == U
    assert state(ws=A[2], wsb=1 << 20) == E    # the workspace aliases v
    # bf16 chunk 16 has no state kernel of its own: segments of 48 tokens are not whole 32- or
    # 64-token chunks, so there is no state pass for them
    assert state(T=96, P=2, chunk=16) == U
    assert b"state-pass" in lib.gla_last_error()

    def dstate(q=A[0], out=A[7], T=256, P=2):
        return lib.gla_chunk_dstate(q, A[3], A[4], out, 1, 1, T, 64, 64, 64, P, gla.GLA_BF16, NUL, 0, NUL)

    assert dstate(q=NUL) == E
    assert dstate(out=NUL) == E
    assert dstate(out=A[4]) == E               # the output aliases do
    assert dstate(P=3) == E

    def fwd_from(seg_in=A[8], o=A[9], ws=WS, wsb=1 << 20):
        return lib.gla_chunk_fwd_from(A[0], A[1], A[2], A[3], seg_in, o, A[10], 1, 1, 256, 64, 64, 64, 2,
                                      gla.GLA_BF16, ws, wsb, NUL)

    assert fwd_from(seg_in=NUL) == E
    assert b"seg_in" in lib.gla_last_error()
    assert fwd_from(o=NUL) == E
    assert fwd_from(o=A[8]) == E               # o aliases seg_in
    assert fwd_from(ws=NUL) == E               # the workspace is required, as for gla_chunk_fwd
    assert fwd_from(wsb=8) == E

    def bwd_from(seg_grad=A[11], dq=A[12], ws=WS, wsb=1 << 20):
        return lib.gla_chunk_bwd_from(A[0], A[1], A[2], A[3], A[4], A[10], A[8], seg_grad, dq, A[13], A[14], A[15],
                                      1, 1, 256, 64, 64, 64, 2, gla.GLA_BF16, ws, wsb, NUL)

    assert bwd_from(seg_grad=NUL) == E
    assert b"seg_grad" in lib.gla_last_error()
    assert bwd_from(dq=NUL) == E
    assert bwd_from(dq=A[11]) == E             # dq aliases seg_grad
    assert bwd_from(ws=NUL) == E


def test_states_first_segments():
    # the order with the incoming states first cuts the segments in two until B*H*P' fills the chip
    # (256 units) or a half would drop below 2 chunks
    f = gla.states_first_segments
    assert f(1, 4, 1 << 20, 64, 64) == 64          # 256 units already
    assert f(1, 16, 16384, 64, 4) == 16            # 64 units -> 256
    assert f(2, 4, 16384, 64, 1) == 32             # 8 units -> 256
    assert f(1, 4, 32768, 64, 8) == 64             # 32 units -> 256
    assert f(1, 1, 256, 16, 4) == 8                # stops at 2 chunks a segment
    assert f(1, 1, 960, 64, 3) == 3                # 5 chunks a segment: no halving
    assert f(4, 64, 4096, 64, 1) == 1
    for B, H, T, C, P in [(1, 2, 4096, 64, 4), (1, 3, 6144, 32, 3), (2, 1, 8192, 16, 2), (1, 1, 64, 16, 1)]:
        Pp = f(B, H, T, C, P)
        assert Pp % P == 0 and (Pp // P) & (Pp // P - 1) == 0 and T % Pp == 0 and (T // Pp) % C == 0
        n = T // Pp // C
        assert B * H * Pp >= 256 or n % 2 == 1 or n // 2 < 2, (B, H, T, C, P, Pp)
    with pytest.raises(ValueError):
        f(1, 1, 250, 16, 4)


def _expected_workspace(B, H, T, dk, dv, C, P, fast=True):
    """The workspace rule of include/gla.h, written out: with fewer than 256 units (b, h, segment)
    each segment is cut into S sub-segments (S a power of two, at least 2 chunks each) until
    B*H*P*S reaches 256; then one int flag per unit and sub-segment, and with S > 1 three float32
    buffers (sub-segment states, their log decays, the scanned states); then, where a unit (b, h,
    segment, sub-segment) splits into pieces of at least 2 chunks, the re-split of flagged units:
    2 + R ints and the same three buffers for R = min(256, units * xmax) slots.  Each region is
    rounded up to 256 bytes."""
    units, nch, S = B * H * P, T // P // C, 1
    while fast and units * S < 256 and nch % (2 * S) == 0 and nch // (2 * S) >= 2:
        S *= 2
    up = lambda n: (n + 255) // 256 * 256  # noqa
    u = units * S
    total = up(4 * u)
    if S > 1:
        total += up(4 * u * dk * dv) + up(4 * u * dk) + up(4 * u * dk * dv)
    nch_u, xmax = nch // S, 1
    while nch_u % (2 * xmax) == 0 and nch_u // (2 * xmax) >= 2:
        xmax *= 2
    R = min(256, u * xmax) if fast and xmax >= 2 else 0
    if R:
        total += up(4 * (2 + R)) + up(4 * R * dk * dv) + up(4 * R * dk) + up(4 * R * dk * dv)
    return total


def test_workspace_size(lib):
    for B, H, T, P, C in [(1, 1, 256, 1, 64), (1, 4, 1 << 20, 64, 64), (3, 5, 64 * 77, 77, 16), (8, 16, 4096, 64, 64),
                          (2, 4, 16384, 1, 64), (1, 4, 32768, 8, 64), (1, 16, 16384, 4, 64), (1, 1, 1024, 4, 32)]:
        for which in (gla.GLA_FWD, gla.GLA_BWD):
            n = lib.gla_workspace_size(which, B, H, T, 128, 256, C, P, gla.GLA_BF16)
            assert n == _expected_workspace(B, H, T, 128, 256, C, P, fast=C != 16), (B, H, T, P, C)
            assert n == gla.workspace_size(which, B, H, T, 128, 256, C, P, torch.bfloat16)
    # the headline workload fills the chip unsplit: flags, then the re-split's 256 slots
    state = 128 * 256 * 4
    assert lib.gla_workspace_size(gla.GLA_BWD, 1, 4, 1 << 20, 128, 256, 64, 64, gla.GLA_BF16) == \
        1024 + 1280 + 256 * (2 * state + 128 * 4)
    # units of 2 chunks do not split further: no re-split region
    assert lib.gla_workspace_size(gla.GLA_FWD, 1, 4, 64 * 128, 128, 256, 64, 64, gla.GLA_BF16) == 1024
    assert lib.gla_workspace_size(gla.GLA_FWD, 1, 1, 250, 64, 64, 64, 4, gla.GLA_BF16) == 0  # T % P
    assert lib.gla_workspace_size(7, 1, 1, 256, 64, 64, 64, 4, gla.GLA_BF16) == 0            # unknown call
    assert lib.gla_workspace_size(gla.GLA_BWD, 1, 1, 256, 48, 64, 64, 4, gla.GLA_BF16) == 0  # no kernel
    with pytest.raises(gla.GLAError):
        gla.workspace_size(gla.GLA_FWD, 1, 1, 250, 64, 64, 64, 4, torch.bfloat16)


def test_binding_checks_every_tensor_against_the_call():
    # the binding derives (B, H, T, dk, dv) from q and v and checks every other tensor against it
    # before anything reaches the library (checked here on host tensors, one helper at a time)
    q = torch.zeros(1, 2, 64, 32, dtype=torch.bfloat16)
    gla._expect(q, "q", (1, 2, 64, 32), torch.bfloat16, q.device)
    with pytest.raises(ValueError):
        gla._expect(q, "k", (1, 2, 64, 16), torch.bfloat16, q.device)      # wrong d_k
    with pytest.raises(TypeError):
        gla._expect(q.float(), "k", (1, 2, 64, 32), torch.bfloat16, q.device)  # fp32 k next to bf16 q
    with pytest.raises(ValueError):
        gla._expect(q[:, :, ::2], "v", (1, 2, 32, 32), torch.bfloat16, q.device)  # not contiguous
    with pytest.raises(ValueError):
        gla._expect(None, "g", (1, 2, 64, 32), torch.float32, q.device)
    gla._expect(None, "h_boundary", (1, 2, 32, 32), torch.float32, q.device, optional=True)
    with pytest.raises(ValueError):
        gla._expect(torch.zeros(1, 2, 64), "g", (1, 2, 64, 32), torch.float32, q.device)  # a per-head gate
    assert gla._seg_shapes(1, 2, 256, 32, 64, 16, 4) == ((1, 2, 16, 32, 64), (1, 2, 4, 32, 64), (1, 2, 4, 32))
    for T, P, C in [(250, 4, 16), (256, 3, 16), (256, 8, 64), (256, 0, 16)]:
        with pytest.raises(ValueError):
            gla._seg_shapes(1, 1, T, 32, 32, C, P)


def test_binding_has_no_cpu_fallback():
    q = torch.zeros(1, 1, 64, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gla.gla_chunk_fwd(q, q, q, torch.zeros(1, 1, 64, 32), chunk=32, P=1)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 16), (32, 64), (128, 256)])
def test_chunk_state_tile_layout(dk, dv):
    # the tiled chunk-state layout of include/gla.h, element by element: (c, j) belongs to lane
    # index L = 16 (j % 16 // 4) + c % 16 of tile (c // 16, j // 16); tiles pair up along dv when
    # dv / 16 is even
    rng = torch.Generator().manual_seed(1)
    dense = torch.randn(2, 3, dk, dv, generator=rng)
    tiled = torch.full((2, 3, dk * dv), float("nan"))
    njb = dv // 16
    for c in range(dk):
        for j in range(dv):
            cb, jb, lane = c // 16, j // 16, 16 * (j % 16 // 4) + c % 16
            if njb % 2 == 0:
                off = (cb * njb + jb - jb % 2) * 256 + 8 * lane + 4 * (jb % 2) + j % 4
            else:
                off = (cb * njb + jb) * 256 + 4 * lane + j % 4
            tiled[:, :, off] = dense[:, :, c, j]
    assert not torch.isnan(tiled).any()  # every offset is taken exactly once
    assert torch.equal(gla.chunk_states_dense(tiled.reshape(2, 3, dk, dv)), dense)
