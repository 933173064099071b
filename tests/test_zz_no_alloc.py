"""gla_chunk_fwd_noalloc (the forward's entry point that allocates nothing) against gla_chunk_fwd,
through the C ABI, on two calls in a row, the second one smaller.  The first call uses a strongly
decaying gate, so every unit's flag in the static scratch is left set; the second uses the default
gate, so the fast kernel must overwrite those flags before the exact kernel reads them.
gla_chunk_fwd cuts these small problems' segments into sub-segments and the no-allocation call
does not, so the two agree to rounding: max|x - r| / max|r| <= 2e-2 (bf16) and 1e-4 (f32)."""
import ctypes

import pytest
import torch

from sequence_state_scan_amd import gla, inputs

pytestmark = pytest.mark.gpu


def _outputs(d, chunk, P):
    B, H, T, dk = d["q"].shape
    dv = d["v"].shape[-1]
    dev, f32 = d["q"].device, torch.float32
    return (torch.full((B, H, T, dv), float("nan"), device=dev, dtype=d["q"].dtype),
            torch.full((B, H, T // chunk, dk, dv), float("nan"), device=dev, dtype=d["q"].dtype),
            torch.full((B, H, P, dk, dv), float("nan"), device=dev, dtype=f32),
            torch.full((B, H, P, dk), float("nan"), device=dev, dtype=f32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_forward_matches_the_workspace_call(dtype):
    if dtype == "bf16":
        cases = [(1, 4, 4096, 128, 256, 64, 4, "strong5"), (2, 1, 1024, 64, 128, 32, 2, "logsigmoid16")]
    else:
        cases = [(1, 3, 1024, 32, 32, 32, 4, "strong5"), (1, 2, 256, 16, 32, 16, 2, "logsigmoid16")]
    for B, H, T, dk, dv, chunk, P, gate in cases:
        d = {n: t.cuda() for n, t in inputs.generate(B, H, T, dk, dv, dtype, 7, False, gate).items()}
        ref = gla.gla_chunk_fwd(d["q"], d["k"], d["v"], d["g"], chunk, P)
        got = gla.gla_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], chunk, P, *_outputs(d, chunk, P))
        torch.cuda.synchronize()
        tol = 2e-2 if dtype == "bf16" else 1e-4
        for name, a, b in zip(("o", "chunk_states", "seg_state", "seg_logdecay"), got, ref):
            a, b = a.double(), b.double()
            assert not torch.isnan(a).any(), (B, H, T, dk, dv, chunk, P, gate, name)
            err = float((a - b).abs().max() / b.abs().max())
            assert err <= tol, (B, H, T, dk, dv, chunk, P, gate, name, err)


def test_noalloc_rejects_more_units_than_its_scratch_holds():
    lib = gla.load_library()
    fake = ctypes.c_void_p(0x1000)
    outs = [ctypes.c_void_p(0x2000 + 0x100 * i) for i in range(4)]
    P = 65537  # B*H*P one above the static scratch
    st = lib.gla_chunk_fwd_noalloc(fake, fake, fake, fake, *outs, 1, 1, P * 16, 32, 32, 16, P, gla.GLA_BF16, None)
    assert st == gla.GLA_ERR_INVALID_ARG
    assert b"static scratch" in lib.gla_last_error()
