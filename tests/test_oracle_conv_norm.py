"""Pins of the oracle's short convolution, L2 norm and gated RMSNorm (CPU).

Library routines (torch CPU conv1d, silu, normalize, rms_norm, sigmoid) serve
as independent references; the streaming and impulse checks pin the tap order
and the rolling-state semantics drawn in the short-convolution diagram of
"Inside Kimi K3" (lei.chat).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F


@pytest.fixture(params=["numpy", "c"])
def conv(request, np_oracle, c_oracle):
    return np_oracle.short_conv_silu if request.param == "numpy" else c_oracle.short_conv_silu


def test_impulse_response_gives_taps_in_reverse(conv):
    """An impulse at t = 0 yields pre-activations w3, w2, w1, w0 at t = 0..3
    (tap 0 multiplies x_{t-3}, tap 3 multiplies x_t), then zero."""
    C = 5
    rng = np.random.default_rng(0)
    w = rng.standard_normal((C, 4))
    x = np.zeros((7, C))
    x[0] = 1.0
    y, _ = conv(x, w)
    pre = np.zeros((7, C))
    pre[0:4] = w[:, ::-1].T
    expect = F.silu(torch.from_numpy(pre)).numpy()
    np.testing.assert_allclose(y, expect, rtol=1e-14, atol=1e-15)


def test_matches_torch_conv1d(conv):
    rng = np.random.default_rng(1)
    T, C = 37, 6
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, 4)) * 0.25
    y, _ = conv(x, w)
    xt = torch.from_numpy(x.T.copy())[None]                 # [1, C, T]
    pre = F.conv1d(F.pad(xt, (3, 0)), torch.from_numpy(w)[:, None, :], groups=C)
    expect = F.silu(pre)[0].T.numpy()
    np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-13)


def test_rolling_state_split_call(conv):
    """conv(x) equals conv(x[:t1]) followed by conv(x[t1:]) seeded with the
    first call's rolling state; the final states agree bitwise."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((40, 4))
    w = rng.standard_normal((4, 4))
    y, st = conv(x, w)
    ya, sa = conv(x[:13], w)
    yb, sb = conv(x[13:], w, sa)
    np.testing.assert_allclose(np.concatenate([ya, yb]), y, rtol=1e-14, atol=1e-15)
    assert np.array_equal(sb, st)
    assert np.array_equal(st, x[-3:].T)


def test_decode_streaming_matches_prefill(conv):
    """One token at a time with the rolling state reproduces the full conv."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((12, 3))
    w = rng.standard_normal((3, 4))
    s0 = rng.standard_normal((3, 3))
    y, st = conv(x, w, s0)
    s = s0
    for t in range(12):
        yt, s = conv(x[t:t + 1], w, s)
        np.testing.assert_allclose(yt[0], y[t], rtol=1e-14, atol=1e-15)
    assert np.array_equal(s, st)


def test_short_sequence_state(conv):
    """With T < 3 the new state mixes the old state and the new inputs."""
    x = np.array([[7.0], [8.0]])
    s0 = np.array([[1.0, 2.0, 3.0]])
    w = np.ones((1, 4))
    _, st = conv(x, w, s0)
    assert np.array_equal(st, np.array([[3.0, 7.0, 8.0]]))
    _, st0 = conv(np.zeros((0, 1)), w, s0)
    assert np.array_equal(st0, s0)


def test_channels_never_mix(conv):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((20, 6))
    w = rng.standard_normal((6, 4))
    y, _ = conv(x, w)
    x2 = x.copy()
    x2[:, 2] += 5.0
    y2, _ = conv(x2, w)
    changed = np.any(y2 != y, axis=0)
    assert list(np.nonzero(changed)[0]) == [2]
    assert y.shape == x.shape            # no sequence shortening


def test_l2norm(np_oracle, c_oracle):
    rng = np.random.default_rng(5)
    u = rng.standard_normal((50, 128)) * 3.0
    for f in (np_oracle.l2norm, c_oracle.l2norm_rows):
        v = f(u, 1e-6)
        norms = np.linalg.norm(v, axis=1)
        # ||v|| = ||u|| / sqrt(||u||^2 + eps)
        nu = np.linalg.norm(u, axis=1)
        np.testing.assert_allclose(norms, nu / np.sqrt(nu ** 2 + 1e-6), rtol=1e-14)
        ref = F.normalize(torch.from_numpy(u), dim=1, eps=0.0).numpy()
        np.testing.assert_allclose(v, ref, rtol=1e-7)


def test_gated_rmsnorm_matches_torch(np_oracle, c_oracle):
    rng = np.random.default_rng(6)
    o = rng.standard_normal((33, 64))
    z = rng.standard_normal((33, 64))
    w = 1.0 + 0.02 * rng.standard_normal(64)
    ot = torch.from_numpy(o)
    ref = (F.rms_norm(ot, (64,), torch.from_numpy(w), eps=1e-6) *
           torch.sigmoid(torch.from_numpy(z))).numpy()
    for f in (np_oracle.gated_rmsnorm, c_oracle.gated_rmsnorm):
        np.testing.assert_allclose(f(o, z, w, 1e-6), ref, rtol=1e-12, atol=1e-14)


def test_gated_rmsnorm_rms_property(c_oracle):
    """Dividing out weight and gate leaves rows of RMS (1 + eps/mean o^2)^-1/2."""
    rng = np.random.default_rng(7)
    o = rng.standard_normal((10, 128))
    z = rng.standard_normal((10, 128))
    w = 1.0 + 0.02 * rng.standard_normal(128)
    y = c_oracle.gated_rmsnorm(o, z, w, 1e-6)
    base = y / (w * (1.0 / (1.0 + np.exp(-z))))
    ms = np.mean(o * o, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(base ** 2, axis=1)),
                               1.0 / np.sqrt(1.0 + 1e-6 / ms), rtol=1e-12)
