"""Pins of the oracle's MXFP8 decoding (CPU), and of the input encoder against it.

The MXFP8 reading (OCP microscaling: E4M3 elements, one E8M0 scale per 32
values) is the plainest one of the pages' "MXFP8 activations" ("Inside Kimi
K3", model at a glance)."""
import numpy as np
import torch

import synth
from oracle import kda_ref as ref


def test_e4m3_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ours = ref.e4m3_value(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.array_equal(ours[~np.isnan(ours)], lib[~np.isnan(lib)])


def test_e4m3_closed_forms():
    v = ref.e4m3_value
    assert v(0x00) == 0.0 and np.signbit(v(0x80)) and v(0x80) == 0.0
    assert v(0x38) == 1.0 and v(0xB8) == -1.0
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0          # largest finite
    assert v(0x08) == 2.0 ** -6                              # smallest normal
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9  # subnormals
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))


def test_e8m0_closed_forms():
    v = ref.e8m0_value
    assert v(127) == 1.0 and v(128) == 2.0 and v(0) == 2.0 ** -127 and v(254) == 2.0 ** 127
    assert np.isnan(v(255))


def test_scales_apply_per_block_of_32():
    codes = np.full((2, 128), 0x38, dtype=np.uint8)          # every element 1.0
    scales = np.array([[120, 121, 122, 123], [127, 127, 0, 254]], dtype=np.uint8)
    out = ref.mxfp8_decode(codes, scales)
    for r in range(2):
        for b in range(4):
            assert np.all(out[r, 32 * b:32 * (b + 1)] == 2.0 ** (int(scales[r, b]) - 127))


def test_encoder_round_trip_within_e4m3_precision():
    """decode(encode(x)) keeps every value to E4M3's relative precision
    (2^-4) once it is at least 2^-6 of its block's largest value; smaller
    values lose at most one subnormal step of the block scale."""
    g = torch.Generator().manual_seed(7)
    x = torch.randn((64, 256), generator=g) * torch.exp2(torch.randint(-20, 20, (64, 1), generator=g).float())
    codes, scales = synth.mxfp8_encode(x)
    back = ref.mxfp8_decode(codes.numpy(), scales.numpy())
    xd = x.double().numpy()
    scale = np.repeat(ref.e8m0_value(scales.numpy()), 32, axis=-1)
    err = np.abs(back - xd)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(xd), 2.0 ** -10 * scale))
    # every block's largest value lands in (224, 448]: the top of E4M3's
    # range, with no saturation
    amax = np.abs(back).reshape(64, 8, 32).max(-1) / ref.e8m0_value(scales.numpy())
    assert np.all((amax >= 224) & (amax <= 448))
