"""Pins of the oracle's gated latent-attention decode step (CPU): closed
forms that the gated multi-head latent attention diagram of "Inside Kimi K3"
(lei.chat) fixes -- one cached token, equal scores, a dominant score, the
gate, and the invariance of softmax to a shift of all scores."""
import numpy as np
import torch


def _setup(seed=0, B=3, H=4, Dk=8, Dv=6, R=10, L=7):
    rng = np.random.default_rng(seed)
    return dict(q=rng.standard_normal((B, H, Dk)), w_uk=rng.standard_normal((H, Dk, R)) * 0.3,
                w_uv=rng.standard_normal((H, Dv, R)) * 0.3, cache=rng.standard_normal((B, L, R)),
                gate=rng.standard_normal((B, H, Dv)))


def test_one_cached_token_returns_its_gated_value(np_oracle):
    """With a single cached latent the weight is 1: y = sigmoid(g) * (W_uv c_0)."""
    a = _setup()
    y = np_oracle.mla_decode(a["q"], a["w_uk"], a["w_uv"], a["cache"], [1, 1, 1], a["gate"])
    for b in range(3):
        for h in range(4):
            v0 = a["w_uv"][h] @ a["cache"][b, 0]
            np.testing.assert_allclose(y[b, h], v0 / (1 + np.exp(-a["gate"][b, h])), rtol=1e-12)


def test_zero_query_averages_the_values(np_oracle):
    """q = 0 makes every score equal: the output is the mean of the values."""
    a = _setup(1)
    L = [7, 3, 5]
    y = np_oracle.mla_decode(np.zeros_like(a["q"]), a["w_uk"], a["w_uv"], a["cache"], L, a["gate"])
    for b in range(3):
        mean_c = a["cache"][b, :L[b]].mean(0)
        for h in range(4):
            expect = (a["w_uv"][h] @ mean_c) * torch.sigmoid(torch.from_numpy(a["gate"][b, h])).numpy()
            np.testing.assert_allclose(y[b, h], expect, rtol=1e-12)


def test_dominant_score_selects_one_token(np_oracle):
    """A query far along one key direction puts (almost) all weight on the
    token with the largest score."""
    a = _setup(2, B=1, H=1)
    c = a["cache"][0]
    k = c @ a["w_uk"][0].T
    q = 200.0 * k[4] / np.linalg.norm(k[4])
    scores = k @ q
    best = int(np.argmax(scores))
    y = np_oracle.mla_decode(q[None, None], a["w_uk"], a["w_uv"], a["cache"], [7], np.zeros((1, 1, 6)),
                             scale=1.0)
    np.testing.assert_allclose(y[0, 0], 0.5 * (a["w_uv"][0] @ c[best]), rtol=1e-6, atol=1e-9)


def test_matches_torch_attention_and_ignores_rows_past_length(np_oracle):
    """Against torch's scaled dot-product attention on the reconstructed keys
    and values (CPU, fp64); cache rows past each length change nothing."""
    a = _setup(3)
    L = [7, 2, 4]
    y = np_oracle.mla_decode(a["q"], a["w_uk"], a["w_uv"], a["cache"], L, a["gate"])
    cache2 = a["cache"].copy()
    for b in range(3):
        cache2[b, L[b]:] = 1e3
    y2 = np_oracle.mla_decode(a["q"], a["w_uk"], a["w_uv"], cache2, L, a["gate"])
    np.testing.assert_array_equal(y, y2)
    for b in range(3):
        c = torch.from_numpy(a["cache"][b, :L[b]])
        for h in range(4):
            k = c @ torch.from_numpy(a["w_uk"][h]).T
            v = c @ torch.from_numpy(a["w_uv"][h]).T
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(a["q"][b, h])[None, None, None], k[None, None], v[None, None])[0, 0, 0]
            expect = o.numpy() * torch.sigmoid(torch.from_numpy(a["gate"][b, h])).numpy()
            np.testing.assert_allclose(y[b, h], expect, rtol=1e-10)
