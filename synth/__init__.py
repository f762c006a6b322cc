"""Seeded synthetic inputs for the KDA token mixer.

This module only draws random numbers: it holds none of the method's
arithmetic, and both the HIP path's tests/bench and the CPU oracle read the
tensors it returns (the oracle after an exact upcast to fp64).

Distributions follow the layer shape the pages draw (96 heads x 128 dims,
projected q/k/v [B, T, 96, 128], rolling conv state [B, 36864, 3], filter banks
[12288, 1, 4], log-decay bounded below by -5).  ``N(0, s)`` means standard
deviation ``s``.  ``beta`` is passed already squashed into (0, 1), which is the
form the layer consumes; the squashing is a property of the input distribution.

Every tensor is drawn by its own ``torch.Generator`` seeded from
``(seed, tensor_id)``, on the device it will live on (host draws for the CPU
tests, device draws for the large GPU workloads), in float32, then rounded to
the I/O dtype with round-to-nearest-even.
"""
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import torch

# tensor ids used to derive per-tensor seeds
TID_X, TID_CONV_W, TID_G, TID_BETA, TID_GATE, TID_NORM_W, TID_S0, TID_CONV_STATE, TID_LENS = range(9)
TID_Q, TID_W_UK, TID_W_UV, TID_CACHE = range(9, 13)


@dataclass(frozen=True)
class PrefillSpec:
    """One prefill workload (shapes and value distributions)."""
    name: str
    H: int
    D: int
    dtype: str                      # "f32" or "bf16" for every per-token tensor
    lengths: Tuple[int, ...] = ()   # fixed sequence lengths (packed); or
    n_seqs: int = 0                 # ... draw n_seqs lengths ~ U[len_lo, len_hi]
    len_lo: int = 0
    len_hi: int = 0
    varlen: bool = False            # pass cu_seqlens (packed) rather than B x T
    chunk: int = 0                  # tokens per chunk; 0 = the library's fastest
    x_std: float = 1.0
    conv_w_std: float = 0.25
    g_lo: float = -5.0
    g_hi: float = 0.0
    beta_mean: float = 0.0          # beta = sigmoid(N(beta_mean, beta_std))
    beta_std: float = 1.0
    gate_std: float = 1.0
    norm_w_std: float = 0.02        # norm weight = 1 + N(0, norm_w_std)
    s0_std: float = 0.0             # 0 -> zero initial state (passed as NULL)
    conv_state_std: float = 0.0     # 0 -> no initial conv state
    seed: int = 1000


@dataclass(frozen=True)
class DecodeSpec:
    name: str
    B: int
    H: int
    D: int
    dtype: str
    steps: int
    x_std: float = 1.0
    conv_w_std: float = 0.25
    g_lo: float = -5.0
    g_hi: float = 0.0
    beta_mean: float = 0.0
    beta_std: float = 1.0
    s0_std: float = 0.1
    conv_state_std: float = 1.0
    gate_std: float = 1.0
    norm_w_std: float = 0.02
    seed: int = 1004


@dataclass(frozen=True)
class MlaSpec:
    """One decode step of gated latent attention: B sequences with up to
    L_max cached 512-wide latents, H heads of 128.  Cached lengths are L_max
    for every sequence unless ``len_lo`` > 0 (then U[len_lo, L_max])."""
    name: str
    B: int
    H: int
    L_max: int
    R: int = 512
    Dh: int = 128
    len_lo: int = 0
    q_std: float = 1.0
    w_std: float = 512 ** -0.5     # up-projections: unit-variance keys and values
    cache_std: float = 1.0
    gate_std: float = 1.0
    seed: int = 3000


# The five workloads of the measurement plan, plus stress variants that make
# the inter-chunk carry visible (with g ~ U(-5, 0) a chunk forgets its
# entering state almost completely).
CONFIGS = {
    0: PrefillSpec("tiny_T256_H2_D64_f32", H=2, D=64, dtype="f32", lengths=(256,), seed=1000),
    1: PrefillSpec("prefill_T4096_H96_D128_bf16", H=96, D=128, dtype="bf16", lengths=(4096,),
                   seed=1001),
    2: PrefillSpec("prefill_T65536_H96_D128_bf16", H=96, D=128, dtype="bf16", lengths=(65536,),
                   seed=1002),
    3: PrefillSpec("varlen_16seq_U512_8192_H96_D128_bf16", H=96, D=128, dtype="bf16", n_seqs=16,
                   len_lo=512, len_hi=8192, varlen=True, s0_std=0.1, seed=1003),
    4: DecodeSpec("decode_B256_H96_D128_bf16_64steps", B=256, H=96, D=128, dtype="bf16", steps=64,
                  seed=1004),
}

# Latent-cache decode step of the global attention layers: the decode batch of
# 256 sequences over a 4096-token cache.
MLA = {
    "decode": MlaSpec("mla_decode_B256_L4096_H96_R512_bf16", B=256, H=96, L_max=4096, seed=3001),
}

STRESS = {
    "slow_decay": PrefillSpec("slow_decay_T4096_H96_D128_bf16", H=96, D=128, dtype="bf16",
                              lengths=(4096,), g_lo=-0.05, s0_std=0.1, seed=2001),
    "long_carry": PrefillSpec("long_carry_T65536_H4_D128_bf16", H=4, D=128, dtype="bf16",
                              lengths=(65536,), g_lo=-2e-5, beta_mean=-6.0, beta_std=0.5,
                              s0_std=0.1, seed=2002),
    # the 1M-token regime: the state carried across 65,536 chunks
    "long_carry_1M": PrefillSpec("long_carry_T1048576_H2_D128_bf16", H=2, D=128, dtype="bf16",
                                 lengths=(1048576,), g_lo=-2e-5, beta_mean=-6.0, beta_std=0.5,
                                 s0_std=0.1, seed=2003),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed: int, tid: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + tid * 7_919 + 17)
    return g


def _normal(shape, std, mean, seed, tid, device, dtype):
    t = torch.randn(shape, generator=_gen(seed, tid, device), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def _uniform(shape, lo, hi, seed, tid, device, dtype):
    t = torch.rand(shape, generator=_gen(seed, tid, device), device=device, dtype=torch.float32)
    t.mul_(hi - lo).add_(lo)
    return t.clamp_(lo, hi).to(dtype)


def seq_lengths(spec: PrefillSpec):
    """Sequence lengths of a prefill spec (drawn on the host for varlen)."""
    if spec.lengths:
        return list(spec.lengths)
    gen = _gen(spec.seed, TID_LENS, "cpu")
    lens = torch.randint(spec.len_lo, spec.len_hi + 1, (spec.n_seqs,), generator=gen)
    return [int(v) for v in lens]


def prefill_inputs(spec: PrefillSpec, device="cpu", lengths=None):
    """Draw every input of one prefill workload.

    Returns a dict of tensors on ``device``:
      x [N, 3HD] (I/O dtype), conv_w [3HD, 4] f32, g [N, H, D], beta [N, H],
      gate [N, H, D], norm_w [D] f32, S0 [S, H, D, D] f32 or None,
      conv_state [S, 3HD, 3] or None, cu (host int64 list of offsets),
    plus ``lengths`` and ``spec``.
    """
    lengths = list(lengths) if lengths is not None else seq_lengths(spec)
    H, D = spec.H, spec.D
    P = 3 * H * D
    N = sum(lengths)
    S = len(lengths)
    dt = TORCH_DTYPE[spec.dtype]
    sd = spec.seed
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    out = dict(spec=spec, lengths=lengths, cu=cu)
    out["x"] = _normal((N, P), spec.x_std, 0.0, sd, TID_X, device, dt)
    out["conv_w"] = _normal((P, 4), spec.conv_w_std, 0.0, sd, TID_CONV_W, device, torch.float32)
    out["g"] = _uniform((N, H, D), spec.g_lo, spec.g_hi, sd, TID_G, device, dt)
    out["beta"] = torch.sigmoid(_normal((N, H), spec.beta_std, spec.beta_mean, sd, TID_BETA,
                                        device, torch.float32)).to(dt)
    out["gate"] = _normal((N, H, D), spec.gate_std, 0.0, sd, TID_GATE, device, dt)
    out["norm_w"] = (1.0 + _normal((D,), spec.norm_w_std, 0.0, sd, TID_NORM_W, device,
                                   torch.float32))
    out["S0"] = (_normal((S, H, D, D), spec.s0_std, 0.0, sd, TID_S0, device, torch.float32)
                 if spec.s0_std > 0 else None)
    out["conv_state"] = (_normal((S, P, 3), spec.conv_state_std, 0.0, sd, TID_CONV_STATE, device,
                                 dt) if spec.conv_state_std > 0 else None)
    return out


def decode_inputs(spec: DecodeSpec, device="cpu", steps=None):
    """Draw the initial states and every step's token inputs of a decode run.

    Returns conv_w [3HD, 4] f32, S0 [B, H, D, D] f32, conv_state [B, 3HD, 3],
    x [steps, B, 3HD], g [steps, B, H, D], beta [steps, B, H],
    gate [steps, B, H, D], norm_w [D] f32.
    """
    steps = spec.steps if steps is None else steps
    B, H, D = spec.B, spec.H, spec.D
    P = 3 * H * D
    dt = TORCH_DTYPE[spec.dtype]
    sd = spec.seed
    return dict(
        spec=spec,
        conv_w=_normal((P, 4), spec.conv_w_std, 0.0, sd, TID_CONV_W, device, torch.float32),
        S0=_normal((B, H, D, D), spec.s0_std, 0.0, sd, TID_S0, device, torch.float32),
        conv_state=_normal((B, P, 3), spec.conv_state_std, 0.0, sd, TID_CONV_STATE, device, dt),
        x=_normal((steps, B, P), spec.x_std, 0.0, sd, TID_X, device, dt),
        g=_uniform((steps, B, H, D), spec.g_lo, spec.g_hi, sd, TID_G, device, dt),
        beta=torch.sigmoid(_normal((steps, B, H), spec.beta_std, spec.beta_mean, sd, TID_BETA,
                                   device, torch.float32)).to(dt),
        gate=_normal((steps, B, H, D), spec.gate_std, 0.0, sd, TID_GATE, device, dt),
        norm_w=1.0 + _normal((D,), spec.norm_w_std, 0.0, sd, TID_NORM_W, device, torch.float32),
    )


def scaled(spec, **kw):
    """A copy of a spec with some fields replaced (smaller T, fewer heads...)."""
    return replace(spec, **kw)


def mla_inputs(spec: MlaSpec, device="cpu", lengths=None):
    """Draw one latent-attention decode step (all bf16 but ``lengths``):
    q [B, H, Dh], w_uk / w_uv [H, Dh, R], cache [B, L_max, R], gate [B, H, Dh]
    (logits), lengths [B] int32 on ``device`` (also as ``lengths_list``)."""
    B, H, L, R, Dh, sd = spec.B, spec.H, spec.L_max, spec.R, spec.Dh, spec.seed
    dt = torch.bfloat16
    if lengths is None:
        if spec.len_lo > 0:
            lengths = torch.randint(spec.len_lo, L + 1, (B,), generator=_gen(sd, TID_LENS, "cpu"))
            lengths = [int(v) for v in lengths]
        else:
            lengths = [L] * B
    return dict(
        spec=spec,
        q=_normal((B, H, Dh), spec.q_std, 0.0, sd, TID_Q, device, dt),
        w_uk=_normal((H, Dh, R), spec.w_std, 0.0, sd, TID_W_UK, device, dt),
        w_uv=_normal((H, Dh, R), spec.w_std, 0.0, sd, TID_W_UV, device, dt),
        cache=_normal((B, L, R), spec.cache_std, 0.0, sd, TID_CACHE, device, dt),
        gate=_normal((B, H, Dh), spec.gate_std, 0.0, sd, TID_GATE, device, dt),
        lengths=torch.tensor(lengths, dtype=torch.int32, device=device),
        lengths_list=list(lengths),
    )


def mxfp8_encode(x: torch.Tensor, block: int = 32):
    """Encode a tensor as MXFP8 along its last axis (OCP microscaling, E4M3
    elements, one E8M0 scale per block of 32): the scale is the smallest power
    of two that brings the block's largest magnitude to at most 448, E4M3's
    largest finite value (so nothing saturates), and the scaled values are
    rounded to E4M3.  Returns (codes uint8 [..., C], scales uint8
    [..., C/32]).  Input preparation only: decoding is the oracle's and the
    kernels' own."""
    x = x.float()
    C = x.shape[-1]
    assert C % block == 0
    xb = x.reshape(*x.shape[:-1], C // block, block)
    amax = xb.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.ceil(torch.log2(amax.clamp_min(2.0 ** -126) / 448.0)),
                    torch.full_like(amax, -127.0)).clamp(-127.0, 127.0)
    y = (xb / torch.exp2(e).unsqueeze(-1)).clamp(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(x.shape)
    scales = (e + 127.0).to(torch.uint8)
    return codes, scales
