"""The seeded generator: determinism, shapes, ranges (CPU)."""
import torch

import synth


def test_prefill_shapes_and_determinism():
    spec = synth.scaled(synth.CONFIGS[1], lengths=(40,), H=3)
    a = synth.prefill_inputs(spec)
    b = synth.prefill_inputs(spec)
    assert a["x"].shape == (40, 3 * 3 * 128) and a["x"].dtype == torch.bfloat16
    assert a["g"].shape == (40, 3, 128) and a["beta"].shape == (40, 3)
    assert a["conv_w"].dtype == torch.float32 and a["conv_w"].shape == (3 * 3 * 128, 4)
    for key in ("x", "conv_w", "g", "beta", "gate", "norm_w"):
        assert torch.equal(a[key], b[key]), key
    assert a["S0"] is None and a["conv_state"] is None
    assert float(a["g"].float().min()) >= -5.0 and float(a["g"].float().max()) <= 0.0
    assert 0.0 < float(a["beta"].float().min()) and float(a["beta"].float().max()) < 1.0


def test_varlen_lengths_in_range():
    spec = synth.CONFIGS[3]
    lens = synth.seq_lengths(spec)
    assert len(lens) == 16 and all(512 <= L <= 8192 for L in lens)
    assert lens == synth.seq_lengths(spec)


def test_decode_shapes():
    spec = synth.scaled(synth.CONFIGS[4], B=2, H=2, steps=3)
    d = synth.decode_inputs(spec)
    assert d["S0"].shape == (2, 2, 128, 128) and d["S0"].dtype == torch.float32
    assert d["conv_state"].shape == (2, 3 * 2 * 128, 3)
    assert d["x"].shape == (3, 2, 768)
