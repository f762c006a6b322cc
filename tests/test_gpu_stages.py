"""Stage parity on the GPU: each C ABI call against the CPU oracle on the same
inputs, at sizes the oracle finishes in seconds that still span several tiles
and a ragged tail, plus the edge cases (empty and very short sequences,
in-place states, strided q/k/v views)."""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_09_amd as kda
from oracle import c_oracle, kda_ref
from tests.kda_testlib import ELEM, TOL, f64, max_abs, rel_l2, report

pytestmark = pytest.mark.gpu
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def _randn(shape, seed, dtype, std=1.0):
    return (torch.randn(shape, generator=_gen(seed), device="cuda") * std).to(dtype)


# ----------------------------------------------------------------- gated norm
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("n", [1, 37, 2000])
def test_gated_norm(dtype, D, n):
    H = 3
    dt = DT[dtype]
    print(f"gated_norm dtype={dtype} D={D} n={n}", flush=True)
    o = _randn((n, H, D), 1, dt)
    z = _randn((n, H, D), 2, dt)
    w = 1.0 + _randn((D,), 3, torch.float32, 0.02)
    y = torch.empty_like(o)
    kda.kda_gated_norm(o, z, w, y, n, H, D)
    ref = c_oracle.gated_rmsnorm(f64(o), f64(z), f64(w))
    assert report("y", f64(y), ref, TOL[dtype], elem=ELEM[dtype]) <= TOL[dtype]
    kda.kda_gated_norm(o, z, w, o, n, H, D)             # in place
    torch.cuda.synchronize()
    assert torch.equal(o, y)


# ----------------------------------------------------------------------- conv
CONV_CASES = [
    # (dtype, D, H, lengths, varlen, with state_in)
    ("f32", 64, 2, [256], False, False),
    ("bf16", 128, 3, [50, 50], False, True),
    ("bf16", 128, 2, [0, 1, 2, 3, 5, 40, 100, 0, 33], True, True),
    ("f32", 128, 2, [70, 1, 0, 65], True, False),
    ("bf16", 64, 5, [129, 31], True, True),
]


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: f"{c[0]}-D{c[1]}-H{c[2]}-{len(c[3])}seq")
def test_conv(case):
    dtype, D, H, lengths, varlen, with_state = case
    print(f"conv case={case}", flush=True)
    dt = DT[dtype]
    P = 3 * H * D
    N, S = sum(lengths), len(lengths)
    x = _randn((max(N, 1), P), 10, dt)[:N].contiguous()
    w = _randn((P, 4), 11, torch.float32, 0.25)
    si = _randn((S, P, 3), 12, dt) if with_state else None
    so = torch.empty((S, P, 3), dtype=dt, device="cuda")
    y = torch.empty_like(x)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    if varlen:
        cu_dev = torch.tensor(cu, dtype=torch.int32, device="cuda")
        kda.kda_conv(x, w, y, 1, N, H, D, conv_state_in=si, conv_state_out=so, cu_seqlens=cu_dev,
                     num_seqs=S)
    else:
        kda.kda_conv(x, w, y, S, N // S, H, D, conv_state_in=si, conv_state_out=so)
    xs, ws = f64(x), f64(w)
    ref_y = np.zeros((N, P))
    ref_s = np.zeros((S, P, 3))
    for s in range(S):
        t0, t1 = cu[s], cu[s + 1]
        ys, ref_s[s] = c_oracle.short_conv_silu(xs[t0:t1], ws, None if si is None else f64(si)[s])
        ys = ys.reshape(t1 - t0, 3, H, D)
        ys[:, :2] = kda_ref.l2norm(ys[:, :2])
        ref_y[t0:t1] = ys.reshape(t1 - t0, P)
    if N:
        assert report("y", f64(y), ref_y, TOL[dtype], elem=ELEM[dtype]) <= TOL[dtype]
    assert np.array_equal(f64(so), ref_s)
    # in-place rolling state gives the same result
    if si is not None:
        s2 = si.clone()
        y2 = torch.empty_like(x)
        if varlen:
            kda.kda_conv(x, w, y2, 1, N, H, D, conv_state_in=s2, conv_state_out=s2,
                         cu_seqlens=cu_dev, num_seqs=S)
        else:
            kda.kda_conv(x, w, y2, S, N // S, H, D, conv_state_in=s2, conv_state_out=s2)
        torch.cuda.synchronize()
        assert torch.equal(s2, so) and torch.equal(y2, y)


# --------------------------------------------------------------------- decode
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_steps(dtype, D):
    B, H, steps = 5, 3, 6
    print(f"decode dtype={dtype} D={D}", flush=True)
    dt = DT[dtype]
    P = 3 * H * D
    w = _randn((P, 4), 20, torch.float32, 0.25)
    cs = _randn((B, P, 3), 21, dt)
    S = _randn((B, H, D, D), 22, torch.float32, 0.1)
    cs_ref, S_ref = f64(cs), f64(S)
    o = torch.empty((B, H, D), dtype=dt, device="cuda")
    for t in range(steps):
        x = _randn((B, P), 100 + t, dt)
        g = (-5.0 * torch.rand((B, H, D), generator=_gen(200 + t), device="cuda")).to(dt)
        beta = torch.sigmoid(torch.randn((B, H), generator=_gen(300 + t), device="cuda")).to(dt)
        kda.kda_decode_step(x, w, cs, g, beta, S, o, B, H, D)
        o_ref, cs_ref, S_ref = c_oracle.kda_decode_step(f64(x), f64(w), cs_ref, f64(g), f64(beta),
                                                        S_ref, H, D)
        assert report(f"o[{t}]", f64(o), o_ref, TOL[dtype]) <= TOL[dtype]
    assert report("S", f64(S), S_ref, TOL[dtype]) <= TOL[dtype]
    assert np.array_equal(f64(cs), cs_ref)


# ------------------------------------------------------------- chunk prefill
def _unit_rows(shape, seed, dtype):
    u = torch.randn(shape, generator=_gen(seed), device="cuda")
    return (u / u.norm(dim=-1, keepdim=True)).to(dtype)


CHUNK_CASES = [
    # (dtype, D, H, lengths, varlen, chunk, with S0, g_lo)
    ("f32", 64, 2, [256], False, 64, False, -5.0),
    ("f32", 64, 2, [200], False, 32, True, -5.0),
    ("f32", 64, 2, [77], False, 16, True, -0.05),
    ("f32", 128, 2, [150], False, 32, True, -5.0),
    ("f32", 128, 1, [40], False, 16, True, -0.05),
    ("bf16", 128, 4, [300], False, 64, True, -5.0),
    ("bf16", 128, 4, [300], False, 32, True, -0.05),
    ("bf16", 64, 4, [190], False, 64, True, -0.05),
    ("bf16", 128, 2, [0, 5, 64, 130, 1, 0, 65], True, 64, True, -0.05),
    ("bf16", 128, 2, [100, 100, 100], False, 64, False, -5.0),
    # 16-token chunks: producer / consumer kernel (ring of 8 LDS slots)
    ("bf16", 128, 4, [300], False, 16, True, -5.0),
    ("bf16", 128, 4, [300], False, 16, True, -0.05),
    ("bf16", 64, 4, [190], False, 16, True, -0.05),
    ("bf16", 128, 2, [0, 5, 64, 130, 1, 0, 65], True, 16, True, -0.05),
    ("bf16", 128, 2, [100, 100, 100], False, 16, False, -5.0),
    ("bf16", 128, 2, [2000], False, 16, True, -0.05),
    # sequences of 2, 3, 2, 6, 8, 16 and 3 chunks: full and short last pairs of
    # the two-chunk inverse batches, and lengths that are exact multiples of 16
    ("bf16", 128, 2, [32, 48, 17, 96, 128, 256, 33], True, 16, True, -5.0),
    ("bf16", 64, 2, [16, 31, 80, 240], True, 16, False, -0.05),
    # 32 sequences x 8 heads = 256 chains: takes the full 128-column slices
    ("bf16", 128, 8, [int(v) for v in np.random.default_rng(5).integers(1, 150, 32)], True, 64,
     True, -0.05),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: f"{c[0]}-D{c[1]}-H{c[2]}-{len(c[3])}seq-C{c[5]}")
def test_chunk_prefill(case):
    dtype, D, H, lengths, varlen, chunk, with_s0, g_lo = case
    print(f"chunk case={case}", flush=True)
    dt = DT[dtype]
    N, S = sum(lengths), len(lengths)
    HD = H * D
    # q | k | v interleaved in one buffer, read through the token stride
    qkv = torch.empty((N, 3 * HD), dtype=dt, device="cuda")
    qkv[:, :HD] = _unit_rows((N, H, D), 30, dt).reshape(N, HD)
    qkv[:, HD:2 * HD] = _unit_rows((N, H, D), 31, dt).reshape(N, HD)
    qkv[:, 2 * HD:] = _randn((N, HD), 32, dt)
    g = (g_lo * torch.rand((N, H, D), generator=_gen(33), device="cuda")).to(dt)
    beta = torch.sigmoid(torch.randn((N, H), generator=_gen(34), device="cuda")).to(dt)
    S0 = _randn((S, H, D, D), 35, torch.float32, 0.1) if with_s0 else None
    o = torch.empty((N, H, D), dtype=dt, device="cuda")
    sT = torch.empty((S, H, D, D), dtype=torch.float32, device="cuda")
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    kw = dict(chunk=chunk, initial_state=S0, final_state=sT)
    if varlen:
        kw.update(cu_seqlens=torch.tensor(cu, dtype=torch.int32, device="cuda"), num_seqs=S)
        B, T = 1, N
    else:
        B, T = S, N // S
    kda.kda_chunk_prefill(qkv[:, :HD], qkv[:, HD:2 * HD], qkv[:, 2 * HD:], 3 * HD, g, beta, o,
                          B, T, H, D, D, **kw)
    q64 = f64(qkv[:, :HD]).reshape(N, H, D)
    k64 = f64(qkv[:, HD:2 * HD]).reshape(N, H, D)
    v64 = f64(qkv[:, 2 * HD:]).reshape(N, H, D)
    g64, b64 = f64(g), f64(beta)
    s064 = f64(S0) if S0 is not None else None
    o_ref = np.zeros((N, H, D))
    S_ref = np.zeros((S, H, D, D))
    for s in range(S):
        t0, t1 = cu[s], cu[s + 1]
        for h in range(H):
            o_ref[t0:t1, h], S_ref[s, h] = c_oracle.gated_delta_rule(
                q64[t0:t1, h], k64[t0:t1, h], v64[t0:t1, h], g64[t0:t1, h], b64[t0:t1, h],
                None if s064 is None else s064[s, h])
    if N:
        assert report("o", f64(o), o_ref, TOL[dtype]) <= TOL[dtype]
    assert report("S_T", f64(sT), S_ref, TOL[dtype]) <= TOL[dtype]
    # same call with the state carried in place gives the same result bitwise
    if S0 is not None:
        st = S0.clone()
        o2 = torch.empty_like(o)
        kw.update(initial_state=st, final_state=st)
        kda.kda_chunk_prefill(qkv[:, :HD], qkv[:, HD:2 * HD], qkv[:, 2 * HD:], 3 * HD, g, beta,
                              o2, B, T, H, D, D, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o2, o) and torch.equal(st, sT)


@pytest.mark.gpu
def test_chunk16_repeatable():
    """The 16-token kernel hands LDS slots between waves through counters; any
    ordering fault shows up as outputs that differ between identical calls.
    Many heads and sequence lengths that wrap the slot ring several times."""
    H, D, lengths = 16, 128, [700, 333, 1000]
    N, S = sum(lengths), len(lengths)
    HD = H * D
    dt = torch.bfloat16
    qkv = torch.empty((N, 3 * HD), dtype=dt, device="cuda")
    qkv[:, :HD] = _unit_rows((N, H, D), 40, dt).reshape(N, HD)
    qkv[:, HD:2 * HD] = _unit_rows((N, H, D), 41, dt).reshape(N, HD)
    qkv[:, 2 * HD:] = _randn((N, HD), 42, dt)
    g = (-0.05 * torch.rand((N, H, D), generator=_gen(43), device="cuda")).to(dt)
    beta = torch.sigmoid(torch.randn((N, H), generator=_gen(44), device="cuda")).to(dt)
    S0 = _randn((S, H, D, D), 45, torch.float32, 0.1)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device="cuda")
    outs = []
    for rep in range(6):
        o = torch.full((N, H, D), float(rep), dtype=dt, device="cuda")
        sT = torch.full((S, H, D, D), float(rep), dtype=torch.float32, device="cuda")
        kda.kda_chunk_prefill(qkv[:, :HD], qkv[:, HD:2 * HD], qkv[:, 2 * HD:], 3 * HD, g, beta, o,
                              1, N, H, D, D, chunk=16, initial_state=S0, final_state=sT,
                              cu_seqlens=cu, num_seqs=S)
        torch.cuda.synchronize()
        outs.append((o, sT))
    for rep in range(1, 6):
        assert torch.equal(outs[rep][0], outs[0][0]), f"o differs between calls (call {rep})"
        assert torch.equal(outs[rep][1], outs[0][1]), f"final state differs between calls (call {rep})"
    # one head against the oracle
    f = lambda t: t.detach().double().cpu().numpy()
    h, s = 5, 2
    t0, t1 = int(cu[s]), int(cu[s + 1])
    o_ref, S_ref = c_oracle.gated_delta_rule(
        f(qkv[t0:t1, h * D:(h + 1) * D]), f(qkv[t0:t1, HD + h * D:HD + (h + 1) * D]),
        f(qkv[t0:t1, 2 * HD + h * D:2 * HD + (h + 1) * D]), f(g[t0:t1, h]), f(beta[t0:t1, h]),
        f(S0[s, h]))
    assert report("o", f(outs[0][0][t0:t1, h]), o_ref, TOL["bf16"]) <= TOL["bf16"]
    assert report("S_T", f(outs[0][1][s, h]), S_ref, TOL["bf16"]) <= TOL["bf16"]


def test_chunk16_bitwise_under_concurrent_load():
    """The slot hand-over must not depend on timing: the 16-token kernel at
    96 heads gives bitwise the same outputs and final states when another
    stream streams memory copies on the same GPU (which changes how its
    waves are scheduled and how long their memory operations take) as when
    it runs alone."""
    H, D, N = 96, 128, 4096
    HD = H * D
    dt = torch.bfloat16
    print("chunk16 under concurrent load: T=4096 H=96", flush=True)
    qkv = torch.empty((N, 3 * HD), dtype=dt, device="cuda")
    qkv[:, :HD] = _unit_rows((N, H, D), 50, dt).reshape(N, HD)
    qkv[:, HD:2 * HD] = _unit_rows((N, H, D), 51, dt).reshape(N, HD)
    qkv[:, 2 * HD:] = _randn((N, HD), 52, dt)
    g = (-5.0 * torch.rand((N, H, D), generator=_gen(53), device="cuda")).to(dt)
    beta = torch.sigmoid(torch.randn((N, H), generator=_gen(54), device="cuda")).to(dt)

    def run(stream):
        o = torch.empty((N, H, D), dtype=dt, device="cuda")
        sT = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")
        kda.kda_chunk_prefill(qkv[:, :HD], qkv[:, HD:2 * HD], qkv[:, 2 * HD:], 3 * HD, g, beta, o,
                              1, N, H, D, D, chunk=16, final_state=sT, stream=stream)
        return o, sT

    main = torch.cuda.current_stream()
    o_ref, s_ref = run(main)
    torch.cuda.synchronize()
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    side = torch.cuda.Stream()   # default priority
    for rep in range(4):
        with torch.cuda.stream(side):
            for _ in range(8):
                dst.copy_(src)
        o, sT = run(main)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"o differs under concurrent load (call {rep})"
        assert torch.equal(sT, s_ref), f"final state differs under concurrent load (call {rep})"
