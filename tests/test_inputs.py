"""The seeded input generator: reproducible, correctly distributed, bf16 rounding is RNE."""
import numpy as np
import pytest
import torch

from sequence_state_scan_amd import inputs


def _rne_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) at the bit level; returns uint16."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def test_same_seed_same_draw_and_order():
    a = inputs.generate(1, 2, 64, 16, 32, "bf16", seed=3, bwd=True)
    b = inputs.generate(1, 2, 64, 16, 32, "bf16", seed=3, bwd=True)
    for n in a:
        assert torch.equal(a[n], b[n])
    c = inputs.generate(1, 2, 64, 16, 32, "bf16", seed=4, bwd=True)
    assert not torch.equal(a["q"], c["q"])
    # do is drawn last: the forward inputs do not depend on whether a backward is drawn
    d = inputs.generate(1, 2, 64, 16, 32, "bf16", seed=3, bwd=False)
    for n in ("q", "k", "v", "g"):
        assert torch.equal(a[n], d[n])


def test_bf16_rounding_is_nearest_even():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32)
    # add exact ties to exercise the even rule
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    got = inputs.to_bf16_rne(x).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, _rne_bf16_bits(x))


def test_gate_distribution():
    g = inputs.generate(1, 1, 4096, 128, 16, "bf16", seed=0)["g"].numpy()
    assert g.dtype == np.float32 and np.all(g <= 0)
    # logsigmoid(N(0,1)) has mean about -0.806; divided by 16
    assert abs(g.mean() - (-0.806 / 16)) < 2e-3
    for variant in ("weak", "zero", "strong", "strong5", "mixed", "scalar"):
        gv = inputs.generate(1, 1, 256, 8, 8, "f32", seed=1, gate=variant)["g"].numpy()
        assert np.all(gv <= 0), variant
    # the strong-decay stress gate: min(-5 + x/4, 0), about -5 per token
    g5 = inputs.generate(1, 1, 4096, 16, 8, "f32", seed=3, gate="strong5")["g"].numpy()
    assert abs(g5.mean() + 5.0) < 0.02 and g5.min() < -6.0
    # per-head scalar decay: one value per token, the same in every channel, drawn like the default
    gs = inputs.generate(1, 2, 512, 16, 8, "f32", seed=2, gate="scalar")["g"].numpy()
    assert np.all(gs == gs[..., :1]) and len(np.unique(gs[0, 0, :, 0])) > 500
    assert abs(gs.mean() - (-0.806 / 16)) < 6e-3
    assert np.all(inputs.generate(1, 1, 8, 8, 8, "f32", gate="zero")["g"].numpy() == 0)


def test_scales_and_dtypes():
    d = inputs.generate(2, 3, 512, 64, 32, "f32", seed=5, bwd=True)
    assert d["q"].dtype == torch.float32 and d["v"].shape == (2, 3, 512, 32)
    assert abs(float(d["k"].std()) - 1 / 8) < 0.01
    b = inputs.generate(1, 1, 16, 16, 16, "bf16", seed=5)
    assert b["q"].dtype == torch.bfloat16 and b["g"].dtype == torch.float32


def test_workloads_are_consistent():
    for w in inputs.WORKLOADS.values():
        assert w.T % w.P == 0 and w.L % w.chunk == 0 and w.dk % w.K == 0, w.name
    assert inputs.HEADLINE in inputs.WORKLOADS


def test_bf16_path_equals_torch_cast_of_f32_draw():
    a = inputs.generate(2, 3, 9000, 16, 32, "bf16", seed=2, bwd=True)
    b = inputs.generate(2, 3, 9000, 16, 32, "f32", seed=2, bwd=True)
    for n in ("q", "k", "v", "do"):
        assert torch.equal(a[n], b[n].to(torch.bfloat16)), n
    assert torch.equal(a["g"], b["g"])


def test_head_slice_regenerates_alone():
    full = inputs.generate(2, 3, 9000, 16, 16, "bf16", seed=7, bwd=True)
    one = inputs.generate_head(2, 3, 9000, 16, 16, 1, 2, "bf16", seed=7, bwd=True)
    for n in full:
        assert torch.equal(full[n][1:2, 2:3], one[n]), n


def test_strong_windows_land_in_the_middle_of_evenly_spread_segments():
    g = inputs.generate(2, 3, 4 * 256, 8, 8, "bf16", 1, False, "logsigmoid16")["g"]
    P, L = 4, 256
    out = inputs.add_strong_windows(g, P, 5, length=64, value=-3.0)
    changed = (out != g).any(dim=-1)  # [B, H, T]
    units = sorted({(b * 3 + h) * P + t // L for b, h, t in changed.nonzero().tolist()})
    assert units == [0, 4, 8, 12, 16]  # i * (24 // 5)
    b, h, p = 0, 1, 0  # unit 4
    seg = out[b, h, p * L:(p + 1) * L]
    assert bool((seg[96:160] == -3.0).all()) and bool((seg[:96] == g[b, h, :96]).all())
    assert bool((out[1, 2] == g[1, 2]).all())  # untouched sequences stay
    assert torch.equal(inputs.add_strong_windows(g, P, 0), g)
    with pytest.raises(ValueError):
        inputs.add_strong_windows(g, P, 25)
