"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
the CPU oracle on exactly the same input values (the oracle reads the GPU's
bf16/fp32 inputs upcast to fp64), restricted to sampled heads when the full
layer is too large for the oracle."""
import numpy as np
import torch

import linear_attention_recurrence_09_amd as kda
import synth
from oracle import c_oracle

TOL = {"f32": 1e-5, "bf16": 2e-2}


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def f64(t):
    return t.detach().float().cpu().double().numpy() if t is not None else None


def report(name, gpu, ref, tol):
    r = rel_l2(gpu, ref)
    print(f"  {name}: rel_l2={r:.3e} max_abs={max_abs(gpu, ref):.3e} (tol {tol:g})", flush=True)
    return r


def head_channels(H, D, heads):
    """Column indices of x/y_qkv for the q, k, v channels of the given heads,
    in the oracle layout part * (len(heads) * D) + j * D + d."""
    cols = []
    for part in range(3):
        for h in heads:
            cols.extend(range(part * H * D + h * D, part * H * D + (h + 1) * D))
    return np.asarray(cols)


def gpu_prefill(inp, chunk=None, device="cuda", prefix=None, final_state=True,
                conv_state_out=True):
    """Run the full prefill path (kda_conv -> kda_chunk_prefill ->
    kda_gated_norm) on the inputs ``synth.prefill_inputs`` drew on the GPU.
    ``prefix`` limits a single-sequence workload to its first tokens."""
    spec = inp["spec"]
    H, D = spec.H, spec.D
    chunk = chunk or spec.chunk
    cu = inp["cu"]
    S = len(cu) - 1
    x, g, beta, gate = inp["x"], inp["g"], inp["beta"], inp["gate"]
    if prefix is not None:
        assert S == 1
        x, g, beta, gate = x[:prefix], g[:prefix], beta[:prefix], gate[:prefix]
        cu = [0, prefix]
    N = x.shape[0]
    if spec.varlen:
        cu_dev = torch.tensor(cu, dtype=torch.int32, device=device)
        kw = dict(cu_seqlens=cu_dev, num_seqs=S, B=1, T=N)
    else:
        kw = dict(B=S, T=N // max(S, 1), num_seqs=S)
    sT = torch.empty((S, H, D, D), dtype=torch.float32, device=device) if final_state else None
    cso = (torch.empty((S, 3 * H * D, 3), dtype=x.dtype, device=device)
           if conv_state_out else None)
    y_qkv, o, y = kda.kda_prefill(x, inp["conv_w"], g, beta, gate, inp["norm_w"], H, D,
                                  conv_state_in=inp["conv_state"], conv_state_out=cso,
                                  initial_state=inp["S0"], final_state=sT, chunk=chunk, **kw)
    return dict(y_qkv=y_qkv, o=o, y=y, S_final=sT, conv_state_out=cso)


def oracle_prefill(inp, heads, prefix=None, snap_t=()):
    """The C oracle over the sampled heads (all sequences)."""
    spec = inp["spec"]
    H, D = spec.H, spec.D
    cols = head_channels(H, D, heads)
    hs = list(heads)
    cu = list(inp["cu"])
    x, g, beta, gate = inp["x"], inp["g"], inp["beta"], inp["gate"]
    if prefix is not None:
        x, g, beta, gate = x[:prefix], g[:prefix], beta[:prefix], gate[:prefix]
        cu = [0, prefix]
    cols_t = torch.as_tensor(cols, device=x.device)
    xs = f64(x.index_select(1, cols_t))
    ws = f64(inp["conv_w"].index_select(0, cols_t))
    gs = f64(g[:, hs])
    bs = f64(beta[:, hs])
    zs = f64(gate[:, hs])
    s0 = f64(inp["S0"][:, hs]) if inp["S0"] is not None else None
    csi = f64(inp["conv_state"].index_select(1, cols_t)) if inp["conv_state"] is not None else None
    return c_oracle.kda_prefill(xs, ws, gs, bs, zs, f64(inp["norm_w"]), cu, len(hs), D,
                                conv_state_in=csi, S0=s0, snap_t=snap_t)


def gpu_heads(out, H, D, heads):
    """Slice a GPU prefill result down to the sampled heads, as fp64 numpy."""
    cols = torch.as_tensor(head_channels(H, D, heads), device=out["o"].device)
    hs = list(heads)
    r = dict(y_qkv=f64(out["y_qkv"].index_select(1, cols)), o=f64(out["o"][:, hs]),
             y=f64(out["y"][:, hs]))
    if out.get("S_final") is not None:
        r["S_final"] = f64(out["S_final"][:, hs])
    if out.get("conv_state_out") is not None:
        r["conv_state_out"] = f64(out["conv_state_out"].index_select(1, cols))
    return r


def compare_prefill(gpu, ref, dtype, keys=("y_qkv", "o", "y", "S_final"), bitwise_state=True):
    tol = TOL[dtype]
    worst = {}
    for key in keys:
        if key in gpu and gpu[key] is not None:
            worst[key] = report(key, gpu[key], ref[key], tol)
            assert worst[key] <= tol, (key, worst[key])
    if bitwise_state and gpu.get("conv_state_out") is not None:
        assert np.array_equal(gpu["conv_state_out"], ref["conv_state_out"]), "conv state differs"
    return worst
