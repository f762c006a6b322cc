"""State hand-over between the calls of the C ABI, and the two bandwidth
kernels at the 1M-token length.

* A prefill of T tokens through kda_conv -> kda_chunk_prefill ->
  kda_gated_norm, whose conv_state_out and final_state then feed K calls of
  kda_decode_step (or one kda_decode_multi call of K tokens), against ONE
  oracle prefill of the T + K tokens: the decode outputs are the oracle's
  outputs at tokens T .. T+K-1, and the states after the last token are the
  oracle's final states ("Inside Kimi K3", KDA short-convolution diagram: the
  autoregressive rolling state of the 3 previous raw inputs; "Animated Kimi
  K3 architecture diagram", local-memory panel: the state carried from one
  step to the next).
* 64 decode steps from given conv and recurrent states against the oracle's
  64-token prefill from the same states (the second route to the decode
  workload's result).
* kda_conv and kda_gated_norm on one sequence of 2^20 tokens at 96 x 128
  (token offsets up to about 77 GB), sampled heads against the oracle over the
  whole length ("Inside Kimi K3", header: the 1M-token context).
"""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_09_amd as kda
import synth
from oracle import c_oracle
from tests.kda_testlib import ELEM, TOL, check_y, f64, head_channels, report

pytestmark = pytest.mark.gpu

# one sequence with incoming conv and recurrent states and slow decay, so
# both states matter for the decoded tokens
_BASE = synth.scaled(synth.CONFIGS[1], H=4, s0_std=0.1, conv_state_std=1.0, g_lo=-0.5,
                     seed=4100)


def _oracle_all(inp, n):
    H, D = inp["spec"].H, inp["spec"].D
    return c_oracle.kda_prefill(f64(inp["x"][:n]), f64(inp["conv_w"]), f64(inp["g"][:n]),
                                f64(inp["beta"][:n]), f64(inp["gate"][:n]), f64(inp["norm_w"]),
                                [0, n], H, D, conv_state_in=f64(inp["conv_state"]),
                                S0=f64(inp["S0"]))


@pytest.mark.parametrize("T,K,dtype,D,multi", [
    (1000, 8, "bf16", 128, False),
    (1000, 8, "bf16", 128, True),
    (2, 5, "bf16", 128, False),      # prefill shorter than the conv window
    (37, 4, "bf16", 64, True),
    (250, 6, "f32", 64, False),
])
def test_prefill_then_decode_equals_longer_prefill(T, K, dtype, D, multi):
    spec = synth.scaled(_BASE, dtype=dtype, D=D, lengths=(T + K,))
    print(f"prefill T={T} then {K} decode tokens ({'one call' if multi else 'K calls'}), "
          f"{dtype} D={D}", flush=True)
    inp = synth.prefill_inputs(spec, device="cuda")
    H = spec.H
    P = 3 * H * D
    cs = torch.empty((1, P, 3), dtype=inp["x"].dtype, device="cuda")
    S = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")
    _, o_pre, y_pre = kda.kda_prefill(inp["x"][:T], inp["conv_w"], inp["g"][:T],
                                      inp["beta"][:T], inp["gate"][:T], inp["norm_w"], H, D,
                                      B=1, T=T, conv_state_in=inp["conv_state"],
                                      conv_state_out=cs, initial_state=inp["S0"], final_state=S)
    od = torch.empty((K, 1, H, D), dtype=inp["x"].dtype, device="cuda")
    if multi:
        om = torch.empty((1, K, H, D), dtype=inp["x"].dtype, device="cuda")
        # (clones: a slice of the packed rows need not be 16-byte aligned)
        kda.kda_decode_multi(inp["x"][T:T + K].unsqueeze(0).clone(), inp["conv_w"], cs,
                             inp["g"][T:T + K].unsqueeze(0).clone(),
                             inp["beta"][T:T + K].unsqueeze(0).clone(), S, 1, K, H, D,
                             o=om, conv_state_out=cs, state_out=S)
        od.copy_(om.transpose(0, 1))
    else:
        for i in range(K):
            kda.kda_decode_step(inp["x"][T + i:T + i + 1].clone(), inp["conv_w"], cs,
                                inp["g"][T + i:T + i + 1].clone(),
                                inp["beta"][T + i:T + i + 1].clone(), S, od[i], 1, H, D)
    torch.cuda.synchronize()
    ref = _oracle_all(inp, T + K)
    tol = TOL[dtype]
    report("prefill o", f64(o_pre), ref["o"][:T], tol)
    check_y("prefill y", f64(y_pre), f64(o_pre), ref["y"][:T], f64(inp["gate"][:T]),
            f64(inp["norm_w"]), dtype)
    report("decoded o", f64(od[:, 0]), ref["o"][T:], tol, block=1)
    report("state after the last token", f64(S), ref["S_final"], tol)
    assert np.array_equal(f64(cs), ref["conv_state_out"]), "conv state differs"


def test_64_decode_steps_equal_prefill_of_the_same_tokens():
    """Decode's 64 steps from given states against the oracle's prefill of the
    same 64 tokens from the same states, for 4 sequences of 4 heads."""
    B, H, D, K = 4, 4, 128, 64
    spec = synth.DecodeSpec("decode_B4_H4_D128_bf16_64steps", B=B, H=H, D=D, dtype="bf16",
                            steps=K, seed=4101)
    print(f"{K} decode steps vs one {K}-token prefill, B={B} H={H}", flush=True)
    d = synth.decode_inputs(spec, device="cuda")
    cs, S = d["conv_state"].clone(), d["S0"].clone()
    od = torch.empty((K, B, H, D), dtype=torch.bfloat16, device="cuda")
    for t in range(K):
        kda.kda_decode_step(d["x"][t], d["conv_w"], cs, d["g"][t], d["beta"][t], S, od[t], B, H, D)
    torch.cuda.synchronize()
    # the same tokens as B packed sequences of K tokens
    x = f64(d["x"].transpose(0, 1).reshape(B * K, -1))
    g = f64(d["g"].transpose(0, 1).reshape(B * K, H, D))
    beta = f64(d["beta"].transpose(0, 1).reshape(B * K, H))
    gate = f64(d["gate"].transpose(0, 1).reshape(B * K, H, D))
    ref = c_oracle.kda_prefill(x, f64(d["conv_w"]), g, beta, gate, f64(d["norm_w"]),
                               [b * K for b in range(B + 1)], H, D,
                               conv_state_in=f64(d["conv_state"]), S0=f64(d["S0"]))
    o_ref = ref["o"].reshape(B, K, H, D).transpose(1, 0, 2, 3)
    report("decoded o (token-major)", f64(od), o_ref, TOL["bf16"], block=1)
    report("states", f64(S), ref["S_final"], TOL["bf16"])
    assert np.array_equal(f64(cs), ref["conv_state_out"]), "conv state differs"


@pytest.mark.slow
def test_conv_2pow20_tokens_sampled_heads():
    N, H, D = 1 << 20, 96, 128
    P = 3 * H * D
    heads = [0, 95]
    print(f"conv T={N} H={H}: filling x on the device", flush=True)
    torch.cuda.empty_cache()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4102)
    x = torch.empty((N, P), dtype=torch.bfloat16, device="cuda").normal_(generator=gen)
    w = torch.empty((P, 4), dtype=torch.float32, device="cuda").normal_(0.0, 0.25, generator=gen)
    y = torch.empty_like(x)
    cso = torch.empty((1, P, 3), dtype=torch.bfloat16, device="cuda")
    kda.kda_conv(x, w, y, 1, N, H, D, conv_state_out=cso)
    torch.cuda.synchronize()
    print("  GPU done; copying the sampled heads", flush=True)
    cols = torch.as_tensor(head_channels(H, D, heads), device="cuda")
    xs = f64(x.index_select(1, cols))
    ys = f64(y.index_select(1, cols))
    cs_gpu = f64(cso.index_select(1, cols))
    ws = f64(w.index_select(0, cols))
    del x, y, cso
    torch.cuda.empty_cache()
    nh = len(heads)
    ref, ref_state = c_oracle.short_conv_silu(xs, ws)
    del xs
    for part in range(2):                      # L2 of q and k per (token, head)
        sl = slice(part * nh * D, (part + 1) * nh * D)
        ref[:, sl] = c_oracle.l2norm_rows(ref[:, sl].reshape(N * nh, D)).reshape(N, nh * D)
    report("y (q|k|v of the sampled heads)", ys, ref, TOL["bf16"], elem=ELEM["bf16"])
    assert np.array_equal(cs_gpu[0], ref_state), "conv state differs"


@pytest.mark.slow
def test_gated_norm_2pow20_tokens_sampled_heads():
    N, H, D = 1 << 20, 96, 128
    heads = [0, 47, 95]
    print(f"gated norm T={N} H={H}: filling inputs on the device", flush=True)
    torch.cuda.empty_cache()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4103)
    o = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda").normal_(generator=gen)
    z = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda").normal_(generator=gen)
    w = 1.0 + 0.02 * torch.randn((D,), generator=gen, device="cuda")
    y = torch.empty_like(o)
    kda.kda_gated_norm(o, z, w, y, N, H, D)
    torch.cuda.synchronize()
    ref = c_oracle.gated_rmsnorm(f64(o[:, heads]), f64(z[:, heads]), f64(w))
    report("y (sampled heads)", f64(y[:, heads]), ref, TOL["bf16"], elem=ELEM["bf16"])
