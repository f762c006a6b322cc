"""MXFP8 chunk prefill on the GPU against the CPU oracle.

The inputs q, k, v and g are drawn in fp32, encoded to MXFP8 (E4M3 codes plus
one E8M0 scale per 32 values) by the input generator, and handed to
kda_chunk_prefill_mxfp8 as bytes.  The oracle decodes the same bytes with its
own MXFP8 decoder and runs the fp64 gated delta rule on the decoded values, so
a wrong decode (scale byte, block index, code table) and a wrong recurrence
both show up against it.  As a second, tighter check the same decoded values,
which bfloat16 holds exactly, go through the bf16 entry point: the two paths
differ only in how the inputs are unpacked, so their outputs agree bitwise."""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_09_amd as kda
import synth
from oracle import c_oracle, kda_ref
from tests.kda_testlib import TOL, f64, report, rel_l2

pytestmark = pytest.mark.gpu
D = 128


def _gen(seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def _inputs(lengths, H, seed, g_lo=-5.0, zero_blocks=False, v_block_scales=False):
    """fp32 q, k (unit rows), v, g in [g_lo, 0], beta, then their MXFP8 form:
    q/k/v codes side by side in one [N, 3*H*128] byte buffer, the four scale
    tensors [N, H, 4] and beta in bf16."""
    N = sum(lengths)
    HD = H * D
    q = torch.randn((N, H, D), generator=_gen(seed), device="cuda")
    k = torch.randn((N, H, D), generator=_gen(seed + 1), device="cuda")
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn((N, H, D), generator=_gen(seed + 2), device="cuda")
    if v_block_scales:   # blocks of 32 values at magnitudes 2^-6 .. 2^6
        e = torch.randint(-6, 7, (N, H, D // 32, 1), generator=_gen(seed + 5), device="cuda")
        v = (v.reshape(N, H, D // 32, 32) * torch.exp2(e.float())).reshape(N, H, D)
    if zero_blocks and N:  # all-zero blocks take the smallest scale byte
        q[::7, :, :32] = 0
        v[::5, :, 64:96] = 0
    g = g_lo * torch.rand((N, H, D), generator=_gen(seed + 3), device="cuda")
    beta = torch.sigmoid(torch.randn((N, H), generator=_gen(seed + 4), device="cuda"))
    codes = torch.empty((N, 3 * HD), dtype=torch.uint8, device="cuda")
    scales = []
    for i, t in enumerate((q, k, v)):
        c, s = synth.mxfp8_encode(t)
        codes[:, i * HD:(i + 1) * HD] = c.reshape(N, HD)
        scales.append(s.contiguous())
    g_codes, g_scales = synth.mxfp8_encode(g)
    return dict(N=N, H=H, codes=codes, qs=scales[0], ks=scales[1], vs=scales[2],
                g=g_codes.contiguous(), gs=g_scales.contiguous(), beta=beta.to(torch.bfloat16))


def _decoded(inp):
    """The oracle's fp64 view of the MXFP8 inputs: [N, H, D] each."""
    N, H = inp["N"], inp["H"]
    HD = H * D
    codes = inp["codes"].cpu().numpy()
    out = []
    for i, sc in enumerate((inp["qs"], inp["ks"], inp["vs"])):
        out.append(kda_ref.mxfp8_decode(codes[:, i * HD:(i + 1) * HD].reshape(N, H, D),
                                        sc.cpu().numpy()))
    out.append(kda_ref.mxfp8_decode(inp["g"].cpu().numpy(), inp["gs"].cpu().numpy()))
    return out


def _run(inp, B, T, cu=None, S0=None, sT=None):
    H, HD = inp["H"], inp["H"] * D
    codes = inp["codes"]
    o = torch.empty((inp["N"], H, D), dtype=torch.bfloat16, device="cuda")
    kw = dict(initial_state=S0, final_state=sT)
    if cu is not None:
        kw.update(cu_seqlens=torch.tensor(cu, dtype=torch.int32, device="cuda"),
                  num_seqs=len(cu) - 1)
    kda.kda_chunk_prefill_mxfp8(codes[:, :HD], inp["qs"], codes[:, HD:2 * HD], inp["ks"],
                                codes[:, 2 * HD:], inp["vs"], 3 * HD, inp["g"], inp["gs"],
                                inp["beta"], o, B, T, H, **kw)
    return o


def _oracle(dec, beta64, cu, heads, s064=None):
    q64, k64, v64, g64 = dec
    S = len(cu) - 1
    o_ref = np.zeros((cu[-1], len(heads), D))
    S_ref = np.zeros((S, len(heads), D, D))
    for s in range(S):
        t0, t1 = cu[s], cu[s + 1]
        for j, h in enumerate(heads):
            o_ref[t0:t1, j], S_ref[s, j] = c_oracle.gated_delta_rule(
                q64[t0:t1, h], k64[t0:t1, h], v64[t0:t1, h], g64[t0:t1, h], beta64[t0:t1, h],
                None if s064 is None else s064[s, h])
    return o_ref, S_ref


CASES = [
    # (name, H, lengths, varlen, with S0, g_lo, zero blocks, v block scales)
    ("fixed-ragged", 2, [100, 100], False, True, -5.0, False, False),
    ("varlen-short", 3, [0, 1, 2, 15, 16, 17, 33, 300, 0, 5], True, False, -5.0, True, False),
    ("slow-decay-scaled-v", 4, [1000], False, True, -1e-3, True, True),
    ("varlen-long", 2, [513, 1, 1200, 64], True, True, -2.0, False, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_chunk_prefill_mxfp8(case):
    name, H, lengths, varlen, with_s0, g_lo, zb, vbs = case
    print(f"mxfp8 chunk case={case}", flush=True)
    inp = _inputs(lengths, H, 700, g_lo, zb, vbs)
    N, S = inp["N"], len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    S0 = (torch.randn((S, H, D, D), generator=_gen(710), device="cuda") * 0.1
          if with_s0 else None)
    sT = torch.empty((S, H, D, D), dtype=torch.float32, device="cuda")
    B, T = (1, N) if varlen else (S, N // S)
    o = _run(inp, B, T, cu if varlen else None, S0, sT)
    dec = _decoded(inp)
    o_ref, S_ref = _oracle(dec, f64(inp["beta"]), cu, list(range(H)), f64(S0))
    if N:
        assert report("o", f64(o), o_ref, TOL["bf16"]) <= TOL["bf16"]
    assert report("S_T", f64(sT), S_ref, TOL["bf16"]) <= TOL["bf16"]

    # the same decoded values through the bf16 entry point (exact in bf16)
    HD = H * D
    qkv = torch.empty((N, 3 * HD), dtype=torch.bfloat16, device="cuda")
    for i in range(3):
        qkv[:, i * HD:(i + 1) * HD] = torch.from_numpy(dec[i].reshape(N, HD)).to(
            torch.bfloat16).cuda()
    g_bf = torch.from_numpy(dec[3]).to(torch.bfloat16).cuda()
    assert np.array_equal(f64(qkv[:, :HD]).reshape(N, H, D), dec[0])
    assert np.array_equal(f64(g_bf), dec[3])
    o_bf = torch.empty_like(o)
    sT_bf = torch.empty_like(sT)
    kw = dict(chunk=16, initial_state=S0, final_state=sT_bf)
    if varlen:
        kw.update(cu_seqlens=torch.tensor(cu, dtype=torch.int32, device="cuda"), num_seqs=S)
    kda.kda_chunk_prefill(qkv[:, :HD], qkv[:, HD:2 * HD], qkv[:, 2 * HD:], 3 * HD, g_bf,
                          inp["beta"], o_bf, B, T, H, D, D, **kw)
    torch.cuda.synchronize()
    same = torch.equal(o, o_bf) and torch.equal(sT, sT_bf)
    r_o = rel_l2(f64(o), f64(o_bf)) if N else 0.0
    r_s = rel_l2(f64(sT), f64(sT_bf))
    print(f"  vs bf16 path: bitwise={same} rel_l2 o={r_o:.2e} S_T={r_s:.2e}", flush=True)
    assert same, (r_o, r_s)

    # the state carried in place gives the same result bitwise
    if S0 is not None:
        st = S0.clone()
        o2 = _run(inp, B, T, cu if varlen else None, st, st)
        torch.cuda.synchronize()
        assert torch.equal(o2, o) and torch.equal(st, sT)


def test_chunk_prefill_mxfp8_full_size_sampled_heads():
    """One sequence of 65536 tokens with 96 heads, the size the throughput
    figure is taken at, in the same launch; the oracle checks three heads."""
    H, T = 96, 65536
    heads = [0, 47, 95]
    print(f"mxfp8 chunk full size T={T} H={H} heads={heads}", flush=True)
    inp = _inputs([T], H, 800, -5.0)
    sT = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")
    o = _run(inp, 1, T, None, None, sT)
    torch.cuda.synchronize()
    sub = dict(inp)
    idx = torch.tensor(heads, device="cuda")
    codes = inp["codes"].reshape(T, 3, H, D)[:, :, idx].reshape(T, 3 * len(heads) * D)
    sub.update(H=len(heads), codes=codes, qs=inp["qs"][:, idx], ks=inp["ks"][:, idx],
               vs=inp["vs"][:, idx], g=inp["g"][:, idx], gs=inp["gs"][:, idx])
    dec = _decoded(sub)
    o_ref, S_ref = _oracle(dec, f64(inp["beta"][:, idx]), np.array([0, T]),
                           list(range(len(heads))))
    assert report("o", f64(o[:, idx]), o_ref, TOL["bf16"]) <= TOL["bf16"]
    assert report("S_T", f64(sT[:, idx]), S_ref, TOL["bf16"]) <= TOL["bf16"]


# --------------------------------------------------------- conv with MXFP8 output
U32 = 2.0 ** -24   # fp32 unit roundoff


def _error_bound(xs, ws, si, cu, u_pre, l2_eps=1e-6):
    """Per-element bound on |kernel's fp32 conv + SiLU (+ L2 for q, k) - exact|,
    before the block scale, from the arithmetic:
      * the 4-tap sum in fp32 is off by at most 4u S, S = sum_j |w_j x_j|
        (u = 2^-24), and SiLU's slope is at most 1.1; SiLU itself (exp and
        reciprocal) adds at most 8u of its value: du = 4.4u S + 8u |SiLU|;
      * the inverse L2 norm carries its own rounding (16u, the sum of 128
        squares and the reciprocal square root) plus the propagated error
        of the squares, ||du||_2 / ||SiLU||_2 relative;
      * the final product rounds once more (u).
    A factor 2 on top.  xs [N, P] and ws [P, 4] as the kernel read them,
    si [S, P, 3] the incoming states or None, cu the sequence offsets,
    u_pre [N, 3, H, D] the oracle's SiLU(conv) before the L2 step."""
    N, P = xs.shape
    absw = np.abs(ws)
    s_abs = np.zeros((N, P))
    for s in range(len(cu) - 1):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        hist = np.zeros((3, P)) if si is None else si[s].T     # oldest first
        xp = np.abs(np.concatenate([hist, xs[t0:t1]], 0))
        for j in range(4):
            s_abs[t0:t1] += absw[:, j] * xp[j:j + t1 - t0]
    s_abs = s_abs.reshape(u_pre.shape)
    du = 4.4 * U32 * s_abs + 8 * U32 * np.abs(u_pre)
    inv = np.ones(u_pre.shape[:3] + (1,))
    inv[:, :2] = 1.0 / np.sqrt(np.square(u_pre[:, :2]).sum(-1, keepdims=True) + l2_eps)
    y = np.abs(u_pre) * inv
    dinv = 16 * U32 + np.sqrt(np.square(du).sum(-1, keepdims=True)) * inv
    dinv[:, 2] = 0.0
    return 2.0 * (inv * du + y * dinv + U32 * y)


def _check_codes(gpu_codes, gpu_scales, ref32, tag, err):
    """GPU MXFP8 encoding of a row set against the oracle's encoding of the
    oracle's values rounded to fp32 (the kernel's precision).  The two agree
    except where a value sits within the kernel's error bound `err` (per
    element, from _error_bound) of a decision: the block's largest magnitude
    within the block's largest bound of a scale boundary 448 * 2^k, or an
    element within its own bound of a midpoint between neighbouring E4M3
    values; there the GPU may take either side, and only those two."""
    rc, rs = kda_ref.mxfp8_encode(ref32)
    gs = gpu_scales.astype(np.int64)
    amax = np.abs(ref32).reshape(*ref32.shape[:-1], -1, 32).max(-1)
    damax = err.reshape(*err.shape[:-1], -1, 32).max(-1)
    near_edge = (kda_ref.e8m0_exponent_for(np.maximum(amax - damax, 0.0))
                 != kda_ref.e8m0_exponent_for(amax + damax))
    bad_scale = (gs != rs) & ~near_edge
    assert not bad_scale.any(), f"{tag}: {bad_scale.sum()} scale bytes differ away from a boundary"
    same_scale = np.repeat(gs == rs, 32, axis=-1)
    gv, rv = kda_ref.e4m3_value(gpu_codes), kda_ref.e4m3_value(rc)
    diff = (gv != rv) & same_scale
    shift = -(np.repeat(rs.astype(np.int64), 32, axis=-1) - 127)
    y = np.ldexp(ref32, shift)
    dy = np.ldexp(err, shift)
    lo = kda_ref.e4m3_round(np.clip(y - dy, -448, 448))
    hi = kda_ref.e4m3_round(np.clip(y + dy, -448, 448))
    near_tie = kda_ref.e4m3_value(lo) != kda_ref.e4m3_value(hi)
    either = (gv == kda_ref.e4m3_value(lo)) | (gv == kda_ref.e4m3_value(hi))
    bad = diff & ~(near_tie & either)
    if bad.any():
        idx = np.argwhere(bad)
        toks = np.unique(idx[:, 0])
        print(f"  {tag}: {bad.sum()} codes differ away from a tie, tokens {toks[:20]} .. "
              f"({len(toks)} tokens), channels {np.unique(idx[:, -1])[:16]}", flush=True)
        for i in idx[:6]:
            i = tuple(i)
            print(f"    at {i}: gpu {gv[i]!r} ref {rv[i]!r} scaled {y[i]!r} window {dy[i]!r} "
                  f"code {int(gpu_codes[i]):#04x}/{int(rc[i]):#04x}", flush=True)
    assert not bad.any(), f"{tag}: codes differ away from a tie"
    n = diff.sum()
    print(f"  {tag}: {n} of {diff.size} codes at a near-tie took the other side; "
          f"{(gs != rs).sum()} scale bytes at a boundary; median window {np.median(dy):.2e} "
          f"(scaled units)", flush=True)
    assert n <= max(4, 1e-4 * diff.size)


CONV_CASES = [
    # (D, H, lengths, varlen, with state_in)
    (128, 3, [50, 50], False, True),
    (128, 2, [0, 1, 2, 3, 5, 40, 300, 0, 33], True, True),
    (64, 5, [129, 31], True, True),
    (128, 4, [1000], False, False),
]


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: f"D{c[0]}-H{c[1]}-{len(c[2])}seq")
def test_conv_mxfp8(case):
    D_, H, lengths, varlen, with_state = case
    print(f"mxfp8 conv case={case}", flush=True)
    P = 3 * H * D_
    N, S = sum(lengths), len(lengths)
    x = (torch.randn((max(N, 1), P), generator=_gen(40), device="cuda")).to(torch.bfloat16)
    x = x[:N].contiguous()
    w = torch.randn((P, 4), generator=_gen(41), device="cuda") * 0.25
    si = (torch.randn((S, P, 3), generator=_gen(42), device="cuda").to(torch.bfloat16)
          if with_state else None)
    so = torch.empty((S, P, 3), dtype=torch.bfloat16, device="cuda")
    codes = torch.empty((N, P), dtype=torch.uint8, device="cuda")
    sc = [torch.empty((N, H, D_ // 32), dtype=torch.uint8, device="cuda") for _ in range(3)]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    kw = dict(conv_state_in=si, conv_state_out=so)
    if varlen:
        kw.update(cu_seqlens=torch.tensor(cu, dtype=torch.int32, device="cuda"), num_seqs=S)
        B, T = 1, N
    else:
        B, T = S, N // S
    kda.kda_conv_mxfp8(x, w, codes, *sc, B, T, H, D_, **kw)
    torch.cuda.synchronize()
    xs, ws = f64(x), f64(w)
    ref_y = np.zeros((N, 3, H, D_))
    ref_s = np.zeros((S, P, 3))
    u_pre = np.zeros((N, 3, H, D_))
    for s in range(S):
        t0, t1 = cu[s], cu[s + 1]
        ys, ref_s[s] = c_oracle.short_conv_silu(xs[t0:t1], ws, None if si is None else f64(si)[s])
        ys = ys.reshape(t1 - t0, 3, H, D_)
        u_pre[t0:t1] = ys
        ys = ys.copy()
        ys[:, :2] = kda_ref.l2norm(ys[:, :2])
        ref_y[t0:t1] = ys
    ref32 = ref_y.astype(np.float32).astype(np.float64)
    err = _error_bound(xs, ws, None if si is None else f64(si), cu, u_pre)
    gc = codes.cpu().numpy().reshape(N, 3, H, D_)
    for part, name in enumerate("qkv"):
        _check_codes(gc[:, part], sc[part].cpu().numpy(), ref32[:, part], name, err[:, part])
    assert np.array_equal(f64(so), ref_s)                 # rolling state: copies of inputs
    # decoded values against the fp64 oracle: within half an E4M3 step
    dec = np.stack([kda_ref.mxfp8_decode(gc[:, p], sc[p].cpu().numpy()) for p in range(3)], 1)
    # an element is off by at most half an E4M3 step of its block, 2^-4 of
    # the block's largest magnitude (or less)
    bar = 0.07 * np.abs(ref_y).max() / max(np.sqrt(np.mean(np.square(ref_y))), 1e-300)
    assert report("y (decoded)", dec, ref_y, 0.05, max_abs_rms=bar) <= 0.05


def test_mxfp8_conv_then_chunk_matches_oracle_chain():
    """kda_conv_mxfp8 -> kda_chunk_prefill_mxfp8 against the oracle's chain:
    conv + L2 in fp64, the oracle's MXFP8 encoding of it (in fp32), decode,
    then the fp64 recurrence."""
    H, T = 4, 777
    P, HD = 3 * H * D, H * D
    x = torch.randn((T, P), generator=_gen(50), device="cuda").to(torch.bfloat16)
    w = torch.randn((P, 4), generator=_gen(51), device="cuda") * 0.25
    g = -5.0 * torch.rand((T, H, D), generator=_gen(52), device="cuda")
    gc, gsc = synth.mxfp8_encode(g)
    gc, gsc = gc.contiguous(), gsc.contiguous()
    beta = torch.sigmoid(torch.randn((T, H), generator=_gen(53), device="cuda")).to(torch.bfloat16)
    codes = torch.empty((T, P), dtype=torch.uint8, device="cuda")
    sc = [torch.empty((T, H, 4), dtype=torch.uint8, device="cuda") for _ in range(3)]
    o = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    sT = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")
    kda.kda_conv_mxfp8(x, w, codes, *sc, 1, T, H, D)
    kda.kda_chunk_prefill_mxfp8(codes[:, :HD], sc[0], codes[:, HD:2 * HD], sc[1],
                                codes[:, 2 * HD:], sc[2], P, gc, gsc, beta, o, 1, T, H,
                                final_state=sT)
    torch.cuda.synchronize()
    ys, _ = c_oracle.short_conv_silu(f64(x), f64(w), None)
    ys = ys.reshape(T, 3, H, D)
    ys[:, :2] = kda_ref.l2norm(ys[:, :2])
    ref32 = ys.astype(np.float32).astype(np.float64)
    q64, k64, v64 = (kda_ref.mxfp8_decode(*kda_ref.mxfp8_encode(ref32[:, p])) for p in range(3))
    g64 = kda_ref.mxfp8_decode(gc.cpu().numpy(), gsc.cpu().numpy())
    b64 = f64(beta)
    o_ref = np.zeros((T, H, D))
    S_ref = np.zeros((1, H, D, D))
    for h in range(H):
        o_ref[:, h], S_ref[0, h] = c_oracle.gated_delta_rule(q64[:, h], k64[:, h], v64[:, h],
                                                             g64[:, h], b64[:, h], None)
    assert report("o", f64(o), o_ref, TOL["bf16"]) <= TOL["bf16"]
    assert report("S_T", f64(sT), S_ref, TOL["bf16"]) <= TOL["bf16"]


def test_conv_mxfp8_full_size_sampled_heads():
    """kda_conv_mxfp8 on the 65,536-token, 96-head prefill workload (the launch
    the MXFP8 step is timed in: nine 4,096-channel blocks, all lanes active),
    three heads (q, k and v channels) against the oracle's encoding."""
    from tests.kda_testlib import head_channels
    spec = synth.CONFIGS[2]
    H, D_ = spec.H, spec.D
    heads = [0, 47, 95]
    print(f"mxfp8 conv full size {spec.name} heads={heads}", flush=True)
    inp = synth.prefill_inputs(spec, device="cuda")
    x, w = inp["x"], inp["conv_w"]
    N, P = x.shape
    codes = torch.empty((N, P), dtype=torch.uint8, device="cuda")
    sc = [torch.empty((N, H, D_ // 32), dtype=torch.uint8, device="cuda") for _ in range(3)]
    kda.kda_conv_mxfp8(x, w, codes, *sc, 1, N, H, D_)
    torch.cuda.synchronize()
    cols = torch.as_tensor(head_channels(H, D_, heads), device="cuda")
    xs, ws = f64(x.index_select(1, cols)), f64(w.index_select(0, cols))
    ys, _ = c_oracle.short_conv_silu(xs, ws, None)
    u_pre = ys.reshape(N, 3, len(heads), D_)
    ys = u_pre.copy()
    ys[:, :2] = kda_ref.l2norm(ys[:, :2])
    ref32 = ys.astype(np.float32).astype(np.float64)
    err = _error_bound(xs, ws, None, [0, N], u_pre)
    del xs
    gc = codes.index_select(1, cols).cpu().numpy().reshape(N, 3, len(heads), D_)
    hidx = torch.tensor(heads, device="cuda")
    for part, name in enumerate("qkv"):
        _check_codes(gc[:, part], sc[part].index_select(1, hidx).cpu().numpy(), ref32[:, part],
                     name, err[:, part])
