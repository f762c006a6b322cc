"""ctypes wrapper of the C fp64 oracle (test infrastructure only).

All arrays are converted to contiguous float64 NumPy arrays; outputs are
allocated here and returned.  Layouts follow ``kda_oracle.c``.
"""
import ctypes

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(_build.ensure_built())
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        d = ctypes.c_double
        _lib.oracle_short_conv_silu.argtypes = [dp, i64, i64, dp, dp, dp, dp]
        _lib.oracle_l2norm_rows.argtypes = [dp, i64, i64, d]
        _lib.oracle_gated_delta_rule.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, dp, dp, dp,
                                                 i64, lp, dp]
        _lib.oracle_gated_rmsnorm.argtypes = [dp, dp, dp, i64, i64, d, dp]
        _lib.oracle_kda_prefill.argtypes = [dp, dp, dp, dp, dp, dp, lp, i64, i64, i64, dp, dp,
                                            dp, dp, d, d, dp, dp, dp, i64, lp, dp]
        _lib.oracle_kda_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, d]
        _lib.oracle_num_threads.restype = ctypes.c_int
        _lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _pl(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


def short_conv_silu(x, w, state_in=None):
    x = _f64(x)
    w = _f64(w)
    T, C = x.shape
    si = None if state_in is None else _f64(state_in)
    y = np.empty((T, C))
    so = np.empty((C, 3))
    lib().oracle_short_conv_silu(_p(x), T, C, _p(w), _p(si), _p(y), _p(so))
    return y, so


def l2norm_rows(u, eps=1e-6):
    u = _f64(u).copy()
    D = u.shape[-1]
    rows = u.size // D
    lib().oracle_l2norm_rows(_p(u), rows, D, eps)
    return u


def gated_delta_rule(q, k, v, g, beta, S0=None, snap_t=()):
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    T, DK = q.shape
    DV = v.shape[1]
    s0 = None if S0 is None else _f64(S0)
    o = np.empty((T, DV))
    S = np.empty((DK, DV))
    st = np.ascontiguousarray(np.asarray(snap_t, dtype=np.int64))
    snaps = np.empty((max(len(st), 1), DK, DV))
    lib().oracle_gated_delta_rule(_p(q), _p(k), _p(v), _p(g), _p(beta), T, DK, DV, _p(s0),
                                  _p(o), _p(S), len(st), _pl(st) if len(st) else None,
                                  _p(snaps))
    if len(st):
        return o, S, snaps[: len(st)]
    return o, S


def gated_rmsnorm(o, z, w, eps=1e-6):
    o, z, w = _f64(o), _f64(z), _f64(w)
    D = o.shape[-1]
    rows = o.size // D
    y = np.empty_like(o)
    lib().oracle_gated_rmsnorm(_p(o), _p(z), _p(w), rows, D, eps, _p(y))
    return y


def kda_prefill(x, w, g, beta, gate, norm_w, cu, H, D, conv_state_in=None, S0=None,
                l2_eps=1e-6, rms_eps=1e-6, snap_t=()):
    """Whole layer over packed sequences; returns a dict of fp64 arrays."""
    x, w, g, beta, gate, norm_w = (_f64(a) for a in (x, w, g, beta, gate, norm_w))
    cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int64))
    S = len(cu) - 1
    N = x.shape[0]
    P = 3 * H * D
    assert x.shape == (N, P) and w.shape == (P, 4)
    csi = None if conv_state_in is None else _f64(conv_state_in)
    s0 = None if S0 is None else _f64(S0)
    cso = np.empty((S, P, 3))
    sf = np.empty((S, H, D, D))
    y_qkv = np.empty((N, P))
    o = np.empty((N, H, D))
    y = np.empty((N, H, D))
    st = np.ascontiguousarray(np.asarray(snap_t, dtype=np.int64))
    snaps = np.empty((S, max(len(st), 1), H, D, D)) if len(st) else None
    lib().oracle_kda_prefill(_p(x), _p(w), _p(g), _p(beta), _p(gate), _p(norm_w), _pl(cu), S,
                             H, D, _p(csi), _p(cso), _p(s0), _p(sf), l2_eps, rms_eps,
                             _p(y_qkv), _p(o), _p(y), len(st),
                             _pl(st) if len(st) else None, _p(snaps))
    out = dict(y_qkv=y_qkv, o=o, y=y, S_final=sf, conv_state_out=cso)
    if len(st):
        out["snaps"] = snaps
    return out


def kda_decode_step(x, w, conv_state, g, beta, state, H, D, l2_eps=1e-6):
    """One decode step; returns (o, new_conv_state, new_state)."""
    x, w, g, beta = (_f64(a) for a in (x, w, g, beta))
    cs = _f64(conv_state).copy()
    S = _f64(state).copy()
    B = x.shape[0]
    o = np.empty((B, H, D))
    lib().oracle_kda_decode_step(_p(x), _p(w), _p(cs), _p(g), _p(beta), _p(S), _p(o), B, H, D,
                                 l2_eps)
    return o, cs, S
