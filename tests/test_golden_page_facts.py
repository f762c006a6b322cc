"""Pin the oracle to the shape, size and bound facts the pages print
(``tests/golden/page_facts.json``, each entry cited), and reproduce the pages'
notebook-trace miniature: output [2, 16, 64], sequential equal to chunkwise,
state shape fixed."""
import json
import os

import numpy as np

from tests import pins

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def fact(name):
    return FACTS[name]["value"]


def test_channel_counts_are_consistent():
    H, D = fact("heads"), fact("head_dim")
    assert fact("conv_state_shape")[1] == 3 * H * D            # combined q|k|v channels
    assert fact("filter_bank_shape") == [H * D, 1, fact("conv_width")]
    assert fact("conv_state_shape")[2] == fact("conv_width") - 1


def test_oracle_conv_state_has_width_minus_one_values(c_oracle):
    rng = np.random.default_rng(0)
    _, st = c_oracle.short_conv_silu(rng.standard_normal((10, 6)), rng.standard_normal((6, 4)))
    assert st.shape == (6, fact("conv_width") - 1)


def test_oracle_honours_log_decay_bound(np_oracle, c_oracle):
    lo = fact("log_decay_min")
    rng = np.random.default_rng(1)
    q = k = np.ones((1, 4)) / 2.0
    v = rng.standard_normal((1, 3))
    S0 = rng.standard_normal((4, 3))
    for f in (np_oracle.gated_delta_rule, c_oracle.gated_delta_rule):
        _, S = f(q, k, v, np.full((1, 4), lo - 3.0), np.zeros(1), S0)
        np.testing.assert_allclose(S, np.exp(lo) * S0, rtol=1e-15)


def test_notebook_trace_miniature(np_oracle, c_oracle):
    B, T, DV = fact("notebook_trace_output_shape")
    DK = 32
    rng = np.random.default_rng(2)
    outs = []
    for b in range(B):
        q = rng.standard_normal((T, DK)); q /= np.linalg.norm(q, axis=1, keepdims=True)
        k = rng.standard_normal((T, DK)); k /= np.linalg.norm(k, axis=1, keepdims=True)
        v = rng.standard_normal((T, DV))
        g = rng.uniform(-5, 0, (T, DK))
        beta = rng.uniform(0, 1, T)
        o_seq, S_seq = c_oracle.gated_delta_rule(q, k, v, g, beta)
        o_chk, S_chk = np_oracle.gated_delta_rule_chunkwise(q, k, v, g, beta, chunk=4)
        assert pins._rel(o_chk, o_seq) < 1e-12
        assert S_seq.shape == (DK, DV) == S_chk.shape
        outs.append(o_seq)
    assert np.stack(outs).shape == (B, T, DV)
