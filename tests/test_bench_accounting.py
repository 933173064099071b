"""The benchmark's algorithmic byte count, checked against a tally of the tensors each call touches.

The roofline figure of bench.py divides alg_bytes(w, "chunk_bwd") by the measured duration of
gla_chunk_bwd, so the count must be exactly what that call reads once and writes once.  The tally
here builds the call's tensors (as torch meta tensors, no memory) from the shapes and dtypes the
binding allocates, and sums their sizes.
"""
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sequence_state_scan_amd import inputs  # noqa: E402


def _nbytes(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="meta").numel() * torch.empty((), dtype=dtype).element_size()


@pytest.mark.parametrize("name", sorted(inputs.WORKLOADS))
def test_chunk_bwd_bytes_are_its_tensors(name):
    w = inputs.WORKLOADS[name]
    e = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    f = torch.float32
    qk, vo = (w.B, w.H, w.T, w.dk), (w.B, w.H, w.T, w.dv)
    seg = (w.B, w.H, w.P, w.dk, w.dv)
    reads = [(qk, e), (qk, e), (vo, e), (qk, f), (vo, e), (seg, f)]  # q, k, v, g, do, seg_in
    writes = [(qk, e), (qk, e), (vo, e), (qk, f), (seg, f)]  # dq, dk, dv, dg, seg_dstate
    tally = sum(_nbytes(s, d) for s, d in reads + writes)
    assert bench.alg_bytes(w, "chunk_bwd") == tally


def test_headline_chunk_bwd_bytes():
    # 4 heads x 2^20 tokens: 3584 bytes per token-head plus 2 x 128 KB per segment state
    w = inputs.WORKLOADS[inputs.HEADLINE]
    assert bench.alg_bytes(w, "chunk_bwd") == 4 * (1 << 20) * 3584 + 4 * 64 * 2 * 128 * 256 * 4 == 15099494400
