"""Pins of the oracle's gated delta rule (CPU only).

Both oracles (C fp64 and NumPy fp64) are checked against closed forms,
invariants and an independent dense-transition construction, then against
each other and against the chunkwise form.
"""
import numpy as np
import pytest

from tests import pins


def _unit(rng, n, d):
    u = rng.standard_normal((n, d))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def _rand_case(seed, T, DK, DV, g_lo=-5.0, s0=True):
    rng = np.random.default_rng(seed)
    q, k = _unit(rng, T, DK), _unit(rng, T, DK)
    v = rng.standard_normal((T, DV))
    g = rng.uniform(g_lo, 0.0, (T, DK))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    S0 = rng.standard_normal((DK, DV)) * 0.1 if s0 else None
    return q, k, v, g, beta, S0


@pytest.fixture(params=["numpy", "c"])
def recurrence(request, np_oracle, c_oracle):
    if request.param == "numpy":
        return np_oracle.gated_delta_rule
    return c_oracle.gated_delta_rule


@pytest.mark.parametrize("pin", pins.ALL_PINS)
def test_pins(recurrence, np_oracle, pin):
    errs = pins.run_all(recurrence, np_oracle.gated_delta_rule_bruteforce)
    assert errs[pin] < pins.TOL, errs


def test_c_matches_numpy(np_oracle, c_oracle):
    args = _rand_case(10, 97, 16, 12)
    o1, S1 = np_oracle.gated_delta_rule(*args)
    o2, S2 = c_oracle.gated_delta_rule(*args)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 64])
@pytest.mark.parametrize("g_lo", [-5.0, -0.05])
def test_chunkwise_equals_sequential(np_oracle, chunk, g_lo):
    """The pages' notebook trace: sequential and chunkwise forms agree."""
    args = _rand_case(11, 100, 16, 8, g_lo=g_lo)
    o1, S1 = np_oracle.gated_delta_rule(*args)
    o2, S2 = np_oracle.gated_delta_rule_chunkwise(*args, chunk=chunk)
    assert pins._rel(o2, o1) < 1e-12
    assert pins._rel(S2, S1) < 1e-12


@pytest.mark.parametrize("T", [1, 5, 77, 300])
def test_state_shape_fixed(recurrence, T):
    """The state keeps shape dk x dv for any sequence length."""
    args = _rand_case(12, T, 8, 6)
    o, S = recurrence(*args)
    assert S.shape == (8, 6)
    assert o.shape == (T, 6)


def test_linearity_in_values_and_state(recurrence):
    """For fixed q, k, g, beta the map (V, S0) -> (O, S_T) is linear."""
    q, k, v1, g, beta, S01 = _rand_case(13, 60, 8, 6)
    rng = np.random.default_rng(14)
    v2 = rng.standard_normal(v1.shape)
    S02 = rng.standard_normal(S01.shape)
    a, b = 0.7, -1.3
    o1, S1 = recurrence(q, k, v1, g, beta, S01)
    o2, S2 = recurrence(q, k, v2, g, beta, S02)
    o3, S3 = recurrence(q, k, a * v1 + b * v2, g, beta, a * S01 + b * S02)
    assert pins._rel(o3, a * o1 + b * o2) < 1e-12
    assert pins._rel(S3, a * S1 + b * S2) < 1e-12


def test_value_columns_independent(recurrence):
    """Columns of the state evolve independently: a subset of value columns
    gives the same columns of O and S_T (only dk is coupled)."""
    q, k, v, g, beta, S0 = _rand_case(15, 50, 8, 10)
    o, S = recurrence(q, k, v, g, beta, S0)
    cols = [1, 4, 7]
    o2, S2 = recurrence(q, k, v[:, cols], g, beta, S0[:, cols])
    assert pins._rel(o2, o[:, cols]) < 1e-13
    assert pins._rel(S2, S[:, cols]) < 1e-13


def test_split_call_hands_over_state(recurrence):
    q, k, v, g, beta, S0 = _rand_case(16, 90, 8, 6)
    o, S = recurrence(q, k, v, g, beta, S0)
    oa, Sa = recurrence(q[:37], k[:37], v[:37], g[:37], beta[:37], S0)
    ob, Sb = recurrence(q[37:], k[37:], v[37:], g[37:], beta[37:], Sa)
    assert pins._rel(np.concatenate([oa, ob]), o) < 1e-13
    assert pins._rel(Sb, S) < 1e-13


def test_identity_padding_steps(recurrence):
    """A step with k = 0, beta = 0, g = 0 leaves the state unchanged (used to
    pad a ragged last chunk)."""
    q, k, v, g, beta, S0 = _rand_case(17, 20, 8, 6)
    o, S = recurrence(q, k, v, g, beta, S0)
    z = np.zeros((5, 8))
    o2, S2 = recurrence(np.concatenate([q, z]), np.concatenate([k, z]),
                        np.concatenate([v, np.ones((5, 6))]), np.concatenate([g, z]),
                        np.concatenate([beta, np.zeros(5)]), S0)
    assert pins._rel(S2, S) < 1e-15
    assert pins._rel(o2[:20], o) < 1e-15


def test_log_decay_clamped_at_minus_five(recurrence):
    """The pages bound the log-decay below by -5; values under it act as -5."""
    q, k, v, g, beta, S0 = _rand_case(18, 30, 8, 6)
    g_low = g.copy()
    g_low[::3] = -9.0
    g_clip = g.copy()
    g_clip[::3] = -5.0
    o1, S1 = recurrence(q, k, v, g_low, beta, S0)
    o2, S2 = recurrence(q, k, v, g_clip, beta, S0)
    assert pins._rel(o1, o2) < 1e-15 and pins._rel(S1, S2) < 1e-15


def test_snapshots(c_oracle, np_oracle):
    args = _rand_case(19, 70, 8, 6)
    o, S, snaps = c_oracle.gated_delta_rule(*args, snap_t=(10, 64, 70))
    for i, t in enumerate((10, 64, 70)):
        _, St = np_oracle.gated_delta_rule(*(a[:t] if a is not None and a.ndim and
                                             a.shape[0] == 70 else a for a in args))
        assert pins._rel(snaps[i], St) < 1e-12
    assert pins._rel(snaps[-1], S) < 1e-15
