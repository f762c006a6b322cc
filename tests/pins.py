"""Checks that pin a gated-delta-rule implementation to facts outside itself.

Each ``pin_*`` takes a recurrence ``f(q, k, v, g, beta, S0) -> (o, S_T)`` and
returns the worst relative error against a closed form, an invariant, or an
independent construction.  They are applied to both oracles, and to mutated
copies of the oracle (``test_oracle_mutations.py``) to show that a plausible
mistake fails at least one of them.

Facts used (pages: "Inside Kimi K3", KDA one-head diagram; "Animated Kimi K3
architecture diagram", local-memory panel), restated:
* the log-decay is bounded below by -5 and acts per key channel (rows of S);
* with write strength 0 the memory only decays;
* the correction makes the written key read back its value exactly when the
  write strength is 1 (delta rule);
* the state keeps the shape dk x dv whatever the length.
"""
import numpy as np

TOL = 1e-9


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.linalg.norm(b), 1e-300)
    return float(np.linalg.norm(a - b) / den)


def _unit(rng, n, d):
    u = rng.standard_normal((n, d))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def pin_pure_decay(f, seed=0, T=23, DK=8, DV=8):
    """beta = 0: S_T = Diag(exp(sum_t g_t)) S0, o_t = (Diag(exp(G_t)) S0)^T q_t.

    g is drawn partly below -5 so a missing clamp shows up; the closed form
    applies the pages' bound to each step.
    """
    rng = np.random.default_rng(seed)
    q, k = _unit(rng, T, DK), _unit(rng, T, DK)
    v = rng.standard_normal((T, DV))
    g = rng.uniform(-7.0, 0.0, (T, DK)) * (rng.uniform(size=(T, DK)) < 0.5) + \
        rng.uniform(-0.3, 0.0, (T, DK))
    beta = np.zeros(T)
    S0 = rng.standard_normal((DK, DV))
    o, S = f(q, k, v, g, beta, S0)
    G = np.cumsum(np.maximum(g, -5.0), axis=0)
    o_ref = np.stack([(np.exp(G[t])[:, None] * S0).T @ q[t] for t in range(T)])
    S_ref = np.exp(G[-1])[:, None] * S0
    return max(_rel(o, o_ref), _rel(S, S_ref))


def pin_beta_one_recall(f, seed=1, T=40, DK=8, DV=6):
    """beta = 1, any decay: after step t the state maps k_t to v_t exactly,
    S_t^T k_t = v_t; with q_t = k_t the read returns v_t."""
    rng = np.random.default_rng(seed)
    k = _unit(rng, T, DK)
    q = k.copy()
    v = rng.standard_normal((T, DV))
    g = rng.uniform(-5.0, 0.0, (T, DK))
    beta = np.ones(T)
    S0 = rng.standard_normal((DK, DV))
    o, S = f(q, k, v, g, beta, S0)
    return max(_rel(o, v), _rel(S.T @ k[-1], v[-1]))


def pin_orthonormal_recall(f, seed=2, DK=8, DV=5):
    """alpha = 1, beta = 1, keys e_{pi(t)} distinct basis vectors (t < dk):
    S_T = sum_t e_t v_t^T + (I - sum_t e_t e_t^T) S0, and querying e_s returns
    v_s (associative recall)."""
    rng = np.random.default_rng(seed)
    T = DK - 2
    perm = rng.permutation(DK)[:T]
    k = np.eye(DK)[perm]
    v = rng.standard_normal((T, DV))
    q = k[::-1].copy()                     # query earlier keys at later steps
    g = np.zeros((T, DK))
    beta = np.ones(T)
    S0 = rng.standard_normal((DK, DV))
    o, S = f(q, k, v, g, beta, S0)
    E = np.zeros((DK, DK))
    E[perm, perm] = 1.0
    S_ref = k.T @ v + (np.eye(DK) - E) @ S0
    # o_t reads key perm[T-1-t]; it is stored iff T-1-t <= t
    o_ref = np.zeros((T, DV))
    for t in range(T):
        s = T - 1 - t
        o_ref[t] = v[s] if s <= t else S0[perm[s]]
    return max(_rel(S, S_ref), _rel(o, o_ref))


def pin_dk1_ema(f, seed=3, T=50):
    """dk = 1 with k = +-1 and constant alpha, beta: the state is a scalar
    exponential moving average, S_t = rho S_{t-1} + beta k v_t with
    rho = alpha (1 - beta), whose sum is the geometric series
    S_T = rho^T S0 + beta sum_t rho^{T-1-t} k_t v_t."""
    rng = np.random.default_rng(seed)
    DV = 3
    k = rng.choice([-1.0, 1.0], size=(T, 1))
    q = rng.choice([-1.0, 1.0], size=(T, 1))
    v = rng.standard_normal((T, DV))
    a, b = 0.9, 0.3
    g = np.full((T, 1), np.log(a))
    beta = np.full(T, b)
    S0 = rng.standard_normal((1, DV))
    o, S = f(q, k, v, g, beta, S0)
    rho = a * (1.0 - b)
    w = rho ** (T - 1 - np.arange(T))
    S_ref = rho ** T * S0 + b * np.sum((w * k[:, 0])[:, None] * v, axis=0, keepdims=True)
    return _rel(S, S_ref)


def pin_bruteforce(f, bruteforce, seed=4, T=7, DK=5, DV=5):
    """T <= 8: the state equals the explicit product of dense transition
    matrices ``bruteforce`` builds (an independent construction)."""
    rng = np.random.default_rng(seed)
    q, k = _unit(rng, T, DK), _unit(rng, T, DK)
    v = rng.standard_normal((T, DV))
    g = rng.uniform(-5.0, 0.0, (T, DK))
    beta = rng.uniform(0.05, 0.95, T)
    S0 = rng.standard_normal((DK, DV))
    o, S = f(q, k, v, g, beta, S0)
    o_ref, S_ref = bruteforce(q, k, v, g, beta, S0)
    return max(_rel(o, o_ref), _rel(S, S_ref))


ALL_PINS = ("pure_decay", "beta_one_recall", "orthonormal_recall", "dk1_ema", "bruteforce")


def run_all(f, bruteforce):
    return {
        "pure_decay": pin_pure_decay(f),
        "beta_one_recall": pin_beta_one_recall(f),
        "orthonormal_recall": pin_orthonormal_recall(f),
        "dk1_ema": pin_dk1_ema(f),
        "bruteforce": pin_bruteforce(f, bruteforce),
    }
