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


# ---------------------------------------------------------------- the oracle's encoder
def test_block_exponent_boundaries():
    """The block exponent is the smallest e with amax <= 448 * 2^e."""
    f = ref.e8m0_exponent_for
    for k in (-20, -3, 0, 5, 30):
        edge = 448.0 * 2.0 ** k
        assert f(edge) == k                                  # exactly at the bound
        assert f(np.nextafter(edge, np.inf)) == k + 1        # just past it
        assert f(edge / 2) == k - 1
        assert f(np.nextafter(edge / 2, np.inf)) == k
    assert f(1.0) == -8                                      # 1 <= 448 / 256 = 1.75
    assert f(1.75) == -8 and f(1.7500001) == -7
    assert f(0.0) == -127                                    # all-zero block
    assert f(1e-45) == -127 and f(2.0 ** 200) == 127         # clamped to E8M0


def test_element_rounding_matches_torch_on_midpoints_and_random_values():
    """Round to nearest, ties to even, against torch's float8_e4m3fn cast:
    every midpoint between neighbouring finite values, the values themselves,
    and random values over the whole range."""
    pos = ref.e4m3_value(np.arange(127))
    mids = (pos[:-1] + pos[1:]) / 2
    rnd = np.random.default_rng(5).uniform(-448, 448, 20000)
    rnd_small = np.random.default_rng(6).uniform(-2.0 ** -5, 2.0 ** -5, 20000)
    for y in (mids, -mids, pos, -pos, rnd, rnd_small):
        lib = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        ours = ref.e4m3_round(y)
        # +0 and -0 both decode to zero; torch keeps the sign of a rounded-down negative
        same = (ours == lib) | ((ours & 0x7F) == 0) & ((lib & 0x7F) == 0)
        assert same.all(), y[~same][:5]


def test_encode_decode_error_bound_and_scale_range():
    """Each decoded value is within half an E4M3 step of the input: 2^-4
    relative for normals, 2^-10 * 2^e absolute in the subnormal range; the
    block's largest magnitude lands in (224, 448] after scaling."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((200, 128)) * np.exp2(rng.integers(-30, 30, (200, 1)))
    x[3, 32:64] = 0.0
    codes, scales = ref.mxfp8_encode(x)
    dec = ref.mxfp8_decode(codes, scales)
    e = np.repeat(scales.astype(np.int64) - 127, 32, axis=-1)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** (e - 10.0))
    assert np.all(np.abs(dec - x) <= bound)
    assert np.all(dec[3, 32:64] == 0) and scales[3, 1] == 0
    amax = np.abs(x).reshape(200, 4, 32).max(-1)
    scaled = amax / 2.0 ** (scales.astype(np.int64) - 127)
    nz = amax > 0
    assert np.all(scaled[nz] <= 448) and np.all(scaled[nz] > 224)


def test_encode_inverts_decode_on_representable_blocks():
    """Blocks built from E4M3 codes with the largest magnitude in (224, 448]
    encode back to the same codes and scale."""
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 0x7E, (50, 64)).astype(np.uint8)
    codes |= (rng.integers(0, 2, (50, 64)) << 7).astype(np.uint8)
    codes[:, 0] = 0x78 | (codes[:, 0] & 0x80)             # 256 in every block of 32
    codes[:, 32] = 0x7E                                    # 448
    scales = rng.integers(100, 150, (50, 2)).astype(np.uint8)
    x = ref.mxfp8_decode(codes, scales)
    c2, s2 = ref.mxfp8_encode(x)
    assert np.array_equal(s2, scales)
    assert np.array_equal(ref.e4m3_value(c2), ref.e4m3_value(codes))
