"""NumPy fp64 oracle of the KDA token mixer -- TEST INFRASTRUCTURE ONLY.

Independent of the C oracle (written separately) and of the HIP library.
Besides the token-by-token definitions it holds two other routes to the same
recurrence, used to pin it:

* :func:`gated_delta_rule_chunkwise` -- the chunkwise form (recurrent across
  chunks, parallel inside one), derived below from the recurrence;
* :func:`gated_delta_rule_bruteforce` -- the state after T steps written as a
  product of explicit dk x dk transition matrices (for tiny T).

It also holds MXFP8 (OCP microscaling: E4M3 elements, one E8M0 scale per 32
values) decoding and encoding, written from the format's definition.

Pages cited:
  [CONV] "Inside Kimi K3" (lei.chat), KDA short-convolution diagram.
  [KDA]  "Inside Kimi K3" (lei.chat), Kimi Delta Attention one-head diagram.
  [MEM]  "Animated Kimi K3 architecture diagram" (github.io), local-memory panel.
  [MLA]  "Inside Kimi K3" (lei.chat), gated multi-head latent attention diagram.
"""
import numpy as np

LOG_DECAY_MIN = -5.0  # [KDA]: the log-decay is bounded below by -5


def silu(u):
    """SiLU / Swish: u * sigmoid(u) ([CONV], [KDA])."""
    return u / (1.0 + np.exp(-u))


def sigmoid(u):
    return 1.0 / (1.0 + np.exp(-u))


# --------------------------------------------------------------------------- conv
def short_conv_silu(x, w, state_in=None):
    """[CONV] causal depthwise conv, width 4, then SiLU.

    x [T, C]; w [C, 4] with tap 0 on x_{t-3} ... tap 3 on x_t; state_in [C, 3]
    (oldest first) or None for zero left padding.  Returns (y [T, C],
    state_out [C, 3]) where state_out holds the last three raw inputs.
    """
    x = np.asarray(x, dtype=np.float64)
    T, C = x.shape
    pad = np.zeros((3, C)) if state_in is None else np.asarray(state_in, np.float64).T
    xt = np.concatenate([pad, x], axis=0)  # xt[tau + 3] = x_tau
    pre = np.zeros((T, C))
    for i in range(4):
        pre += w[:, i][None, :] * xt[i: i + T]
    return silu(pre), xt[T: T + 3].T.copy()


def l2norm(u, eps=1e-6):
    """[KDA] u / sqrt(sum u^2 + eps) over the last axis."""
    u = np.asarray(u, dtype=np.float64)
    return u / np.sqrt(np.sum(u * u, axis=-1, keepdims=True) + eps)


def gated_rmsnorm(o, z, w, eps=1e-6):
    """[KDA] head RMSNorm times a sigmoid gate, per row over the last axis."""
    o = np.asarray(o, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o * r * np.asarray(w, np.float64) * sigmoid(np.asarray(z, np.float64))


# --------------------------------------------------------------------- recurrence
def decay(g):
    """alpha = exp(g) with g clamped to [-5, 0] ([KDA])."""
    return np.exp(np.clip(np.asarray(g, np.float64), LOG_DECAY_MIN, 0.0))


def gated_delta_rule(q, k, v, g, beta, S0=None, snap_t=()):
    """[KDA][MEM] token-by-token gated delta rule for one head.

    Decay first (Sbar = Diag(alpha) S), then probe and correct
    (e = v - Sbar^T k), write (S = Sbar + beta k e^T), read (o = S^T q).
    Returns (o [T, DV], S_T [DK, DV]) and, if snap_t is given, the states
    after each requested prefix length.
    """
    T, DK = q.shape
    DV = v.shape[1]
    S = np.zeros((DK, DV)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, DV))
    snaps = {}
    a = decay(g)
    for t in range(T):
        Sbar = a[t][:, None] * S
        e = v[t] - Sbar.T @ k[t]
        S = Sbar + beta[t] * np.outer(k[t], e)
        o[t] = S.T @ q[t]
        if t + 1 in snap_t:
            snaps[t + 1] = S.copy()
    if snap_t:
        return o, S, np.stack([snaps[s] for s in snap_t])
    return o, S


def gated_delta_rule_chunkwise(q, k, v, g, beta, S0=None, chunk=64):
    """Chunkwise form of the same recurrence ([KDA]: recurrent across chunks,
    parallel within a chunk).  Plain fp64 with pairwise decays.

    Within a chunk with entering state S0 and inclusive local cumulative
    log-decay G_r = sum_{i<=r} g_i (per key channel):
      A_kk[r,s] = sum_c k_rc k_sc exp(G_rc - G_sc)     for s <  r
      A_qk[r,s] = sum_c q_rc k_sc exp(G_rc - G_sc)     for s <= r
      U = (I + diag(beta) A_kk)^{-1} diag(beta) (V - (K*exp(G)) S0)
      O = (Q*exp(G)) S0 + A_qk U
      S_C = diag(exp(G_C)) S0 + (K*exp(G_C - G))^T U
    Row r of U is beta_r e_r.  A partial last chunk is simply shorter.
    """
    T, DK = q.shape
    DV = v.shape[1]
    S = np.zeros((DK, DV)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, DV))
    gc = np.clip(np.asarray(g, np.float64), LOG_DECAY_MIN, 0.0)
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        Q, K, V, b = q[c0:c1], k[c0:c1], v[c0:c1], beta[c0:c1]
        G = np.cumsum(gc[c0:c1], axis=0)
        L = c1 - c0
        diff = G[:, None, :] - G[None, :, :]          # [r, s, c] = G_r - G_s
        lower = np.tril(np.ones((L, L), dtype=bool), -1)
        ldiag = np.tril(np.ones((L, L), dtype=bool), 0)
        E = np.exp(np.where(ldiag[:, :, None], diff, 0.0))  # only s <= r used
        Akk = np.where(lower, np.einsum("rc,sc,rsc->rs", K, K, E), 0.0)
        Aqk = np.where(ldiag, np.einsum("rc,sc,rsc->rs", Q, K, E), 0.0)
        gam = np.exp(G)
        rhs = b[:, None] * (V - (K * gam) @ S)
        U = np.linalg.solve(np.eye(L) + b[:, None] * Akk, rhs)
        o[c0:c1] = (Q * gam) @ S + Aqk @ U
        S = np.exp(G[-1])[:, None] * S + (K * np.exp(G[-1][None, :] - G)).T @ U
    return o, S


def gated_delta_rule_bruteforce(q, k, v, g, beta, S0=None):
    """State after T steps as explicit transition products (tiny T only).

    One step is S_t = T_t S_{t-1} + beta_t k_t v_t^T with the dk x dk matrix
    T_t = (I - beta_t k_t k_t^T) Diag(alpha_t); hence
      S_T = (T_T ... T_1) S_0 + sum_s (T_T ... T_{s+1}) beta_s k_s v_s^T
    and o_t = S_t^T q_t.  Built with dense matrix products in fp64.
    """
    T, DK = q.shape
    DV = v.shape[1]
    S0 = np.zeros((DK, DV)) if S0 is None else np.asarray(S0, np.float64)
    a = decay(g)
    Tm = [(np.eye(DK) - beta[t] * np.outer(k[t], k[t])) @ np.diag(a[t]) for t in range(T)]
    o = np.zeros((T, DV))
    for t in range(T):  # state after t+1 tokens, built from scratch each time
        prod = np.eye(DK)
        for s in range(t, -1, -1):
            prod = prod @ Tm[s]
        St = prod @ S0
        for s in range(t + 1):
            after = np.eye(DK)
            for r in range(t, s, -1):
                after = after @ Tm[r]
            St = St + after @ (beta[s] * np.outer(k[s], v[s]))
        o[t] = St.T @ q[t]
    return o, St if T else S0.copy()


# -------------------------------------------------------------------- layer level
def kda_prefill(x, w, g, beta, gate, norm_w, cu, H, D, conv_state_in=None, S0=None,
                l2_eps=1e-6, rms_eps=1e-6, chunk=None):
    """Whole layer over packed sequences, same layout as the C oracle.

    x [N, 3HD] (q|k|v, head-major inside each part), w [3HD, 4], g [N, H, D],
    beta [N, H], gate [N, H, D], norm_w [D], cu [S+1].  chunk=None runs the
    sequential recurrence; an integer runs the chunkwise form instead.
    """
    x = np.asarray(x, np.float64)
    N, P = x.shape
    S = len(cu) - 1
    y_qkv = np.zeros((N, P))
    cso = np.zeros((S, P, 3))
    o = np.zeros((N, H, D))
    y = np.zeros((N, H, D))
    sf = np.zeros((S, H, D, D))
    for s in range(S):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        si = None if conv_state_in is None else conv_state_in[s]
        ys, cso[s] = short_conv_silu(x[t0:t1], w, si)
        ys = ys.reshape(t1 - t0, 3, H, D)
        ys[:, 0] = l2norm(ys[:, 0], l2_eps)
        ys[:, 1] = l2norm(ys[:, 1], l2_eps)
        y_qkv[t0:t1] = ys.reshape(t1 - t0, P)
        for h in range(H):
            s0 = None if S0 is None else S0[s, h]
            args = (ys[:, 0, h], ys[:, 1, h], ys[:, 2, h], g[t0:t1, h], beta[t0:t1, h], s0)
            if chunk is None:
                oh, Sh = gated_delta_rule(*args)
            else:
                oh, Sh = gated_delta_rule_chunkwise(*args, chunk=chunk)
            o[t0:t1, h] = oh
            sf[s, h] = Sh
            y[t0:t1, h] = gated_rmsnorm(oh, gate[t0:t1, h], norm_w, rms_eps)
    return dict(y_qkv=y_qkv, o=o, y=y, S_final=sf, conv_state_out=cso)


def kda_decode_step(x, w, conv_state, g, beta, state, H, D, l2_eps=1e-6):
    """[CONV][KDA] one decode step for B sequences; returns (o, conv_state', S')."""
    x = np.asarray(x, np.float64)
    B, P = x.shape
    o = np.zeros((B, H, D))
    cs_new = np.zeros((B, P, 3))
    S_new = np.array(state, dtype=np.float64)
    for b in range(B):
        yb, cs_new[b] = short_conv_silu(x[b][None, :], w, conv_state[b])
        u = yb.reshape(3, H, D)
        qb, kb, vb = l2norm(u[0], l2_eps), l2norm(u[1], l2_eps), u[2]
        for h in range(H):
            ob, S_new[b, h] = gated_delta_rule(qb[h][None], kb[h][None], vb[h][None],
                                               g[b, h][None], np.array([beta[b, h]]),
                                               state[b, h])
            o[b, h] = ob[0]
    return o, cs_new, S_new


def mla_decode(q, w_uk, w_uv, cache, lengths, gate, scale=None):
    """[MLA] one new token per sequence of gated multi-head latent attention,
    read over the latent cache, straight from the diagram's moves: every
    cached latent c_i is expanded into a key k_i = W_uk c_i and a value
    v_i = W_uv c_i per head; the new token's query attends to all of them
    (causal softmax of q . k_i, with the new token's own latent already in the
    cache); the head output is the weighted sum of the values, times the
    full-rank sigmoid gate.

    q [B, H, Dk], w_uk [H, Dk, R], w_uv [H, Dv, R], cache [B, Lmax, R],
    lengths [B] (cached tokens per sequence, >= 1), gate [B, H, Dv] logits.
    The diagram prints no score scale; 1/sqrt(Dk) is taken.  Returns
    y [B, H, Dv].
    """
    q = np.asarray(q, np.float64)
    B, H, Dk = q.shape
    Dv = w_uv.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(Dk)
    y = np.zeros((B, H, Dv))
    for b in range(B):
        c = np.asarray(cache[b, :lengths[b]], np.float64)          # [L, R]
        for h in range(H):
            k = c @ np.asarray(w_uk[h], np.float64).T              # [L, Dk]
            v = c @ np.asarray(w_uv[h], np.float64).T              # [L, Dv]
            s = scale * (k @ q[b, h])                              # [L]
            p = np.exp(s - s.max())
            p /= p.sum()
            o = p @ v
            y[b, h] = o * sigmoid(np.asarray(gate[b, h], np.float64))
    return y


# ------------------------------------------------------------------ MXFP8 inputs
# The pages quantise activations to MXFP8 ("Inside Kimi K3", model at a
# glance: MXFP4 weights, MXFP8 activations from SFT onward) without spelling
# the format out.  Read as the OCP microscaling format: 8-bit E4M3 elements
# sharing one power-of-two E8M0 scale per block of 32 consecutive values.

def e4m3_value(code):
    """Value of an E4M3 byte: sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent 0 encodes subnormals m/8 * 2^-6; no infinities; the two
    codes with all exponent and mantissa bits set are NaN."""
    code = np.asarray(code, dtype=np.int64)
    s = (code >> 7) & 1
    e = (code >> 3) & 15
    m = code & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def e8m0_value(code):
    """Value of an E8M0 scale byte: 2^(code - 127); code 255 is NaN."""
    code = np.asarray(code, dtype=np.int64)
    return np.where(code == 255, np.nan, 2.0 ** (code.astype(np.float64) - 127))


def mxfp8_decode(codes, scales, block=32):
    """MXFP8 tensor to fp64: codes [..., C] (E4M3 bytes), scales [..., C/block]
    (E8M0 bytes, one per block of `block` consecutive values of the last
    axis); value = e4m3(code) * e8m0(scale of its block)."""
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    C = codes.shape[-1]
    assert C % block == 0 and scales.shape[-1] == C // block
    return e4m3_value(codes) * np.repeat(e8m0_value(scales), block, axis=-1)


# Non-negative finite E4M3 magnitudes by code (0x00 .. 0x7E), ascending.
_E4M3_POS = e4m3_value(np.arange(127))


def e8m0_exponent_for(amax):
    """Block exponent of the MXFP8 encoding: the smallest integer e with
    amax <= 448 * 2^e (448 is E4M3's largest finite value, so no element of
    the block saturates), clamped to E8M0's range [-127, 127]; an all-zero
    block takes -127.  With amax = f * 2^E, f in [0.5, 1) and 448 =
    0.875 * 2^9, that is e = E - 9 when f <= 0.875 and E - 8 otherwise."""
    amax = np.asarray(amax, dtype=np.float64)
    f, E = np.frexp(amax)
    e = np.where(f <= 0.875, E - 9, E - 8)
    e = np.where(amax > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def e4m3_round(y):
    """E4M3 code of y (|y| <= 448), rounded to the nearest representable
    value, ties to the even code (the one whose lowest mantissa bit is 0).
    The sign goes into bit 7; zero gives code 0."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    assert np.all(a <= 448.0), "scaled value outside E4M3's finite range"
    hi = np.searchsorted(_E4M3_POS, a, side="left")        # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == _E4M3_POS[hi], hi, np.where(pick_hi, hi, lo))
    return np.where((y < 0) & (code != 0), code | 0x80, code).astype(np.uint8)


def mxfp8_encode(x, block=32):
    """MXFP8 encoding along the last axis: per block of `block` consecutive
    values, the E8M0 scale byte e + 127 with e from :func:`e8m0_exponent_for`
    of the block's largest magnitude, and each value's E4M3 code of x / 2^e
    (exact division by a power of two, then round to nearest even).  Returns
    (codes uint8 [..., C], scales uint8 [..., C/block])."""
    x = np.asarray(x, dtype=np.float64)
    C = x.shape[-1]
    assert C % block == 0
    xb = x.reshape(*x.shape[:-1], C // block, block)
    e = e8m0_exponent_for(np.abs(xb).max(axis=-1))
    codes = e4m3_round(np.ldexp(xb, -e[..., None])).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)
