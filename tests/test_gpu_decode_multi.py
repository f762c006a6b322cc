"""kda_decode_multi on the GPU against the oracle's one-token decode step
applied token after token: outputs of all K tokens, the states after each
sequence's n_tokens, the rollback protocol (outputs only, then the accepted
tokens in place), K = 1 against kda_decode_step, and the batch of 256
sequences x 96 heads compared on sampled sequences."""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_09_amd as kda
from oracle import c_oracle
from tests.kda_testlib import TOL, f64, report

pytestmark = pytest.mark.gpu
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def _inputs(B, K, H, D, dt, seed=0):
    """Decode-workload distributions: S ~ N(0, 0.1), conv state and x ~ N(0, 1),
    conv taps ~ N(0, 0.25), g ~ U(-5, 0), beta = sigmoid(N(0, 1))."""
    P = 3 * H * D
    r = lambda shape, s, std=1.0: torch.randn(shape, generator=_gen(seed + s), device="cuda") * std
    return dict(
        x=r((B, K, P), 1).to(dt),
        w=r((P, 4), 2, 0.25),
        cs=r((B, P, 3), 3).to(dt),
        g=(-5.0 * torch.rand((B, K, H, D), generator=_gen(seed + 4), device="cuda")).to(dt),
        beta=torch.sigmoid(r((B, K, H), 5)).to(dt),
        S=r((B, H, D, D), 6, 0.1),
    )


def _oracle(inp, H, D, n, seqs=None):
    """Token-by-token oracle; returns o [B, K, H, D] and, per sequence b, the
    conv and recurrent states after its first n[b] tokens."""
    n = np.asarray(n)
    if seqs is not None:
        idx = torch.tensor(list(seqs), device="cuda")
        inp = {k: (v if k == "w" else v.index_select(0, idx)) for k, v in inp.items()}
        n = n[list(seqs)]
    x, g, beta, cs, S, w = (f64(inp[k]) for k in ("x", "g", "beta", "cs", "S", "w"))
    B, K = x.shape[:2]
    o = np.zeros((B, K, H, D))
    cs_snap, S_snap = cs.copy(), S.copy()
    for t in range(K):
        o[:, t], cs, S = c_oracle.kda_decode_step(x[:, t], w, cs, g[:, t], beta[:, t], S, H, D)
        for b in range(B):
            if n[b] == t + 1:
                cs_snap[b], S_snap[b] = cs[b], S[b]
    return o, cs_snap, S_snap


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("K", [1, 2, 3, 5, 8])
def test_decode_multi_vs_oracle(dtype, D, K):
    B, H = 6, 3
    print(f"decode_multi dtype={dtype} D={D} K={K}", flush=True)
    dt = DT[dtype]
    inp = _inputs(B, K, H, D, dt, seed=10 * K + D)
    n = np.array([0, K, 1, K // 2, K, max(K - 1, 0)], dtype=np.int32)
    n_dev = torch.from_numpy(n).cuda()
    o = torch.empty((B, K, H, D), dtype=dt, device="cuda")
    S_out = torch.empty_like(inp["S"])
    cs_out = torch.empty_like(inp["cs"])
    kda.kda_decode_multi(inp["x"], inp["w"], inp["cs"], inp["g"], inp["beta"], inp["S"], B, K, H,
                         D, o=o, conv_state_out=cs_out, state_out=S_out, n_tokens=n_dev)
    o_ref, cs_ref, S_ref = _oracle(inp, H, D, n)
    tol = TOL[dtype]
    for t in range(K):
        assert report(f"o[{t}]", f64(o[:, t]), o_ref[:, t], tol) <= tol
    assert report("S_out", f64(S_out), S_ref, tol) <= tol
    assert np.array_equal(f64(cs_out), cs_ref)
    # sequences that take in no token keep their states bitwise
    assert torch.equal(S_out[0], inp["S"][0]) and torch.equal(cs_out[0], inp["cs"][0])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_multi_rollback(dtype):
    """Check K drafted tokens with the states untouched, then take in the
    accepted prefix of each sequence in place."""
    B, H, D, K = 5, 2, 128, 4
    print(f"decode_multi rollback dtype={dtype}", flush=True)
    dt = DT[dtype]
    inp = _inputs(B, K, H, D, dt, seed=77)
    S0, cs0 = inp["S"].clone(), inp["cs"].clone()
    o = torch.empty((B, K, H, D), dtype=dt, device="cuda")
    kda.kda_decode_multi(inp["x"], inp["w"], inp["cs"], inp["g"], inp["beta"], inp["S"], B, K, H,
                         D, o=o)
    torch.cuda.synchronize()
    assert torch.equal(inp["S"], S0) and torch.equal(inp["cs"], cs0)   # nothing written back
    accepted = np.array([4, 0, 2, 3, 1], dtype=np.int32)
    kda.kda_decode_multi(inp["x"], inp["w"], inp["cs"], inp["g"], inp["beta"], inp["S"], B, K, H,
                         D, conv_state_out=inp["cs"], state_out=inp["S"],
                         n_tokens=torch.from_numpy(accepted).cuda())
    ref_in = dict(inp, S=S0, cs=cs0)
    o_ref, cs_ref, S_ref = _oracle(ref_in, H, D, accepted)
    tol = TOL[dtype]
    assert report("o", f64(o), o_ref, tol) <= tol
    assert report("S (in place)", f64(inp["S"]), S_ref, tol) <= tol
    assert np.array_equal(f64(inp["cs"]), cs_ref)
    # one call with o and the states: the same outputs and states
    S1, cs1 = S0.clone(), cs0.clone()
    o1 = torch.empty_like(o)
    kda.kda_decode_multi(inp["x"], inp["w"], cs1, inp["g"], inp["beta"], S1, B, K, H, D, o=o1,
                         conv_state_out=cs1, state_out=S1,
                         n_tokens=torch.from_numpy(accepted).cuda())
    torch.cuda.synchronize()
    assert torch.equal(o1, o) and torch.equal(S1, inp["S"]) and torch.equal(cs1, inp["cs"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_multi_k1_matches_decode_step(dtype):
    B, H, D = 4, 3, 128
    print(f"decode_multi K=1 vs decode_step dtype={dtype}", flush=True)
    dt = DT[dtype]
    inp = _inputs(B, 1, H, D, dt, seed=5)
    o = torch.empty((B, 1, H, D), dtype=dt, device="cuda")
    S_out, cs_out = torch.empty_like(inp["S"]), torch.empty_like(inp["cs"])
    kda.kda_decode_multi(inp["x"], inp["w"], inp["cs"], inp["g"], inp["beta"], inp["S"], B, 1, H,
                         D, o=o, conv_state_out=cs_out, state_out=S_out)
    S1, cs1 = inp["S"].clone(), inp["cs"].clone()
    o1 = torch.empty((B, H, D), dtype=dt, device="cuda")
    kda.kda_decode_step(inp["x"][:, 0].contiguous(), inp["w"], cs1, inp["g"][:, 0].contiguous(),
                        inp["beta"][:, 0].contiguous(), S1, o1, B, H, D)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert report("o", f64(o[:, 0]), f64(o1), tol) <= tol
    assert report("S", f64(S_out), f64(S1), tol) <= tol
    assert torch.equal(cs_out, cs1)


def test_decode_multi_batch_256_sampled():
    """256 sequences x 96 heads x 128, 4 tokens each, bf16: sampled sequences
    against the oracle."""
    B, H, D, K = 256, 96, 128, 4
    print("decode_multi B=256 H=96 D=128 K=4 bf16", flush=True)
    dt = torch.bfloat16
    inp = _inputs(B, K, H, D, dt, seed=900)
    n = np.random.default_rng(3).integers(0, K + 1, B).astype(np.int32)
    o = torch.empty((B, K, H, D), dtype=dt, device="cuda")
    S_out = torch.empty_like(inp["S"])
    cs_out = torch.empty_like(inp["cs"])
    kda.kda_decode_multi(inp["x"], inp["w"], inp["cs"], inp["g"], inp["beta"], inp["S"], B, K, H,
                         D, o=o, conv_state_out=cs_out, state_out=S_out,
                         n_tokens=torch.from_numpy(n).cuda())
    seqs = [0, 1, 77, 200, 255]
    o_ref, cs_ref, S_ref = _oracle(inp, H, D, n, seqs=seqs)
    tol = TOL["bf16"]
    assert report("o (sampled)", f64(o[seqs]), o_ref, tol) <= tol
    assert report("S (sampled)", f64(S_out[seqs]), S_ref, tol) <= tol
    assert np.array_equal(f64(cs_out[seqs]), cs_ref)
