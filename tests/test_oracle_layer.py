"""Layer-level oracle checks (CPU): C vs NumPy drivers, varlen, decode vs
prefill, and the pages' notebook-trace miniature."""
import numpy as np
import pytest

from tests import pins


def _layer_inputs(seed, lengths, H, D, s0=True, conv_state=True):
    rng = np.random.default_rng(seed)
    N = sum(lengths)
    P = 3 * H * D
    S = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return dict(
        x=rng.standard_normal((N, P)),
        w=rng.standard_normal((P, 4)) * 0.25,
        g=rng.uniform(-5.0, 0.0, (N, H, D)),
        beta=1.0 / (1.0 + np.exp(-rng.standard_normal((N, H)))),
        gate=rng.standard_normal((N, H, D)),
        norm_w=1.0 + 0.02 * rng.standard_normal(D),
        cu=cu,
        conv_state_in=rng.standard_normal((S, P, 3)) if conv_state else None,
        S0=rng.standard_normal((S, H, D, D)) * 0.1 if s0 else None,
    )


def _call(mod, inp, H, D, **kw):
    return mod.kda_prefill(inp["x"], inp["w"], inp["g"], inp["beta"], inp["gate"],
                           inp["norm_w"], inp["cu"], H, D, conv_state_in=inp["conv_state_in"],
                           S0=inp["S0"], **kw)


@pytest.mark.parametrize("lengths", [[33], [5, 0, 17, 2, 40]])
def test_c_driver_matches_numpy_driver(np_oracle, c_oracle, lengths):
    H, D = 2, 8
    inp = _layer_inputs(0, lengths, H, D)
    a = _call(np_oracle, inp, H, D)
    b = _call(c_oracle, inp, H, D)
    for key in ("y_qkv", "o", "y", "S_final", "conv_state_out"):
        np.testing.assert_allclose(b[key], a[key], rtol=1e-11, atol=1e-12, err_msg=key)


def test_numpy_chunked_driver_matches(np_oracle):
    H, D = 2, 8
    inp = _layer_inputs(1, [70, 9], H, D)
    a = _call(np_oracle, inp, H, D)
    b = _call(np_oracle, inp, H, D, chunk=16)
    for key in ("o", "y", "S_final"):
        assert pins._rel(b[key], a[key]) < 1e-12, key


def test_varlen_equals_separate_calls(c_oracle):
    H, D = 2, 8
    lengths = [11, 30, 4]
    inp = _layer_inputs(2, lengths, H, D)
    packed = _call(c_oracle, inp, H, D)
    cu = inp["cu"]
    for s in range(len(lengths)):
        t0, t1 = cu[s], cu[s + 1]
        one = dict(x=inp["x"][t0:t1], w=inp["w"], g=inp["g"][t0:t1], beta=inp["beta"][t0:t1],
                   gate=inp["gate"][t0:t1], norm_w=inp["norm_w"],
                   cu=np.array([0, t1 - t0], np.int64),
                   conv_state_in=inp["conv_state_in"][s:s + 1], S0=inp["S0"][s:s + 1])
        r = _call(c_oracle, one, H, D)
        np.testing.assert_array_equal(r["o"], packed["o"][t0:t1])
        np.testing.assert_array_equal(r["S_final"][0], packed["S_final"][s])


def test_prefill_snapshots(c_oracle):
    H, D = 2, 8
    inp = _layer_inputs(3, [50], H, D)
    full = _call(c_oracle, inp, H, D, snap_t=(20, 50))
    part = dict(inp)
    for key in ("x", "g", "beta", "gate"):
        part[key] = inp[key][:20]
    part["cu"] = np.array([0, 20], np.int64)
    r = _call(c_oracle, part, H, D)
    np.testing.assert_allclose(full["snaps"][0, 0], r["S_final"][0], rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(full["snaps"][0, 1], full["S_final"][0])


@pytest.mark.parametrize("impl", ["numpy", "c"])
def test_decode_steps_equal_prefill(np_oracle, c_oracle, impl):
    """Several decode steps from (conv state, S) equal one prefill of the same
    tokens from the same states: the rolling conv state and the recurrent state
    are the whole context of a sequence."""
    mod = np_oracle if impl == "numpy" else c_oracle
    B, H, D, steps = 3, 2, 8, 6
    rng = np.random.default_rng(4)
    P = 3 * H * D
    w = rng.standard_normal((P, 4)) * 0.25
    cs = rng.standard_normal((B, P, 3))
    S = rng.standard_normal((B, H, D, D)) * 0.1
    xs = rng.standard_normal((steps, B, P))
    gs = rng.uniform(-5, 0, (steps, B, H, D))
    bs = 1 / (1 + np.exp(-rng.standard_normal((steps, B, H))))
    cs_d, S_d = cs.copy(), S.copy()
    o_d = []
    for t in range(steps):
        o, cs_d, S_d = mod.kda_decode_step(xs[t], w, cs_d, gs[t], bs[t], S_d, H, D)
        o_d.append(o)
    o_d = np.stack(o_d, axis=1)                          # [B, steps, H, D]
    for b in range(B):
        r = c_oracle.kda_prefill(xs[:, b], w, gs[:, b], bs[:, b], np.zeros((steps, H, D)),
                                 np.ones(D), [0, steps], H, D, conv_state_in=cs[b:b + 1],
                                 S0=S[b:b + 1])
        np.testing.assert_allclose(o_d[b], r["o"], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(S_d[b], r["S_final"][0], rtol=1e-12, atol=1e-13)
        np.testing.assert_array_equal(cs_d[b], r["conv_state_out"][0])


def test_decode_c_matches_numpy(np_oracle, c_oracle):
    B, H, D = 2, 3, 8
    rng = np.random.default_rng(5)
    P = 3 * H * D
    args = (rng.standard_normal((B, P)), rng.standard_normal((P, 4)),
            rng.standard_normal((B, P, 3)), rng.uniform(-5, 0, (B, H, D)),
            rng.uniform(0, 1, (B, H)), rng.standard_normal((B, H, D, D)))
    a = np_oracle.kda_decode_step(*args, H, D)
    b = c_oracle.kda_decode_step(*args, H, D)
    for x, y in zip(a, b):
        np.testing.assert_allclose(y, x, rtol=1e-12, atol=1e-13)
