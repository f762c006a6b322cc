"""kda_mla_decode on the GPU against the oracle's gated latent-attention decode
step: every head count the kernel is built for, ragged cache lengths across
tile and split boundaries, a near one-hot softmax, a running maximum that
moves on later tiles, many tiles per split, clamped lengths, workspace reuse
and determinism, and the 256-sequence x 4096-token decode workload compared
on sampled sequences."""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_09_amd as kda
import synth
from oracle import kda_ref
from tests.kda_testlib import TOL, f64, report

pytestmark = pytest.mark.gpu
TOL_BF16 = TOL["bf16"]


def _run(inp, ws=None, lengths=None):
    s = inp["spec"]
    y = torch.empty((s.B, s.H, s.Dh), dtype=torch.bfloat16, device="cuda")
    kda.kda_mla_decode(inp["q"], inp["w_uk"], inp["w_uv"], inp["cache"],
                       inp["lengths"] if lengths is None else lengths, inp["gate"], y, s.B, s.H,
                       s.L_max, workspace=ws)
    torch.cuda.synchronize()
    return y


def _oracle(inp, seqs=None, lengths=None):
    lengths = list(inp["lengths_list"] if lengths is None else lengths)
    q, cache, gate = inp["q"], inp["cache"], inp["gate"]
    if seqs is not None:
        idx = torch.tensor(list(seqs), device=q.device)
        q, cache, gate = (t.index_select(0, idx) for t in (q, cache, gate))
        lengths = [lengths[i] for i in seqs]
    return kda_ref.mla_decode(f64(q), f64(inp["w_uk"]), f64(inp["w_uv"]), f64(cache),
                              np.asarray(lengths), f64(gate))


@pytest.mark.parametrize("H", [16, 32, 48, 64, 80, 96])
def test_mla_vs_oracle(H):
    """Cache lengths 1, one tile, one tile + 1, a ragged tail and the full
    cache; with 5 sequences every tile is its own split."""
    print(f"mla H={H}", flush=True)
    spec = synth.MlaSpec(f"mla_H{H}", B=5, H=H, L_max=200, seed=3100 + H)
    inp = synth.mla_inputs(spec, device="cuda", lengths=[1, 32, 33, 95, 200])
    y = _run(inp)
    assert report("y", f64(y), _oracle(inp), TOL_BF16) <= TOL_BF16


def test_mla_peaked_softmax():
    """Queries 6x larger: the softmax is close to one-hot, so a wrong running
    maximum or rescaling across tiles shows at once."""
    print("mla peaked softmax", flush=True)
    spec = synth.MlaSpec("mla_peaked", B=3, H=96, L_max=300, q_std=6.0, seed=3201)
    inp = synth.mla_inputs(spec, device="cuda", lengths=[70, 129, 300])
    y = _run(inp)
    assert report("y", f64(y), _oracle(inp), TOL_BF16) <= TOL_BF16


def test_mla_running_max_moves_on_later_tiles():
    """The kernel moves a head's softmax reference only when a tile's max
    exceeds it by more than 2^8: cached latents that grow 16-fold along the
    sequence (the max jumps by more than that on later tiles, so U is
    rescaled mid-split) and latents that shrink (only the first tile moves
    it).  64 sequences of 640 latents: 4 splits of 5 tiles each."""
    print("mla running max: growing and shrinking latents", flush=True)
    spec = synth.MlaSpec("mla_grow", B=64, H=96, L_max=640, seed=3601)
    inp = synth.mla_inputs(spec, device="cuda")
    t = torch.arange(640, device="cuda", dtype=torch.float32)
    grow = 1.0 + 15.0 * t / 639.0
    fac = torch.ones((64, 640), device="cuda")
    fac[0::2] = grow
    fac[1::2] = grow.flip(0)
    inp["cache"] = (inp["cache"].float() * fac[:, :, None]).to(torch.bfloat16)
    y = _run(inp)
    seqs = [0, 1, 62, 63]
    assert report("y (sampled)", f64(y[seqs]), _oracle(inp, seqs=seqs), TOL_BF16) <= TOL_BF16


def test_mla_many_tiles_per_split():
    """64 sequences split 4 ways: each split runs its online softmax over up
    to 5 tiles of 32 tokens; sampled sequences (the longest included)."""
    print("mla B=64 L_max=640", flush=True)
    spec = synth.MlaSpec("mla_B64", B=64, H=96, L_max=640, len_lo=1, seed=3301)
    lens = synth.mla_inputs(spec, device="cpu")["lengths_list"]
    lens[5] = 640
    inp = synth.mla_inputs(spec, device="cuda", lengths=lens)
    y = _run(inp)
    seqs = [0, 5, 31, 63]
    assert report("y (sampled)", f64(y[seqs]), _oracle(inp, seqs=seqs), TOL_BF16) <= TOL_BF16


def test_mla_lengths_are_clamped():
    """Lengths below 1 read one cached token, above L_max read L_max."""
    print("mla clamped lengths", flush=True)
    spec = synth.MlaSpec("mla_clamp", B=4, H=32, L_max=64, seed=3401)
    inp = synth.mla_inputs(spec, device="cuda", lengths=[0, -7, 64 + 5, 40])
    y = _run(inp)
    assert report("y", f64(y), _oracle(inp, lengths=[1, 1, 64, 40]), TOL_BF16) <= TOL_BF16


def test_mla_workspace_reuse_and_determinism():
    """One workspace serves a large call then a smaller one; repeated calls
    give bitwise the same result as calls with a fresh workspace."""
    print("mla workspace reuse", flush=True)
    big = synth.mla_inputs(synth.MlaSpec("mla_big", B=40, H=96, L_max=256, len_lo=1,
                                         seed=3501), device="cuda")
    small = synth.mla_inputs(synth.MlaSpec("mla_small", B=3, H=96, L_max=100, len_lo=1,
                                           seed=3502), device="cuda")
    n = kda.kda_mla_decode_workspace_bytes(40, 96, 256)
    assert n >= kda.kda_mla_decode_workspace_bytes(3, 96, 100)
    ws = torch.full((n,), 0x7f, dtype=torch.uint8, device="cuda")   # non-zero garbage
    y_big = _run(big, ws=ws)
    y_small = _run(small, ws=ws)
    assert torch.equal(y_big, _run(big)) and torch.equal(y_small, _run(small))
    assert torch.equal(_run(small, ws=ws), y_small)
    assert report("y small", f64(y_small), _oracle(small), TOL_BF16) <= TOL_BF16


def test_mla_empty_batch():
    spec = synth.MlaSpec("mla_empty", B=0, H=96, L_max=8)
    inp = synth.mla_inputs(spec, device="cuda")
    y = torch.empty((0, 96, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(1, dtype=torch.uint8, device="cuda")
    kda.kda_mla_decode(inp["q"], inp["w_uk"], inp["w_uv"], inp["cache"], inp["lengths"],
                       inp["gate"], y, 0, 96, 8, workspace=ws)
    torch.cuda.synchronize()


def test_mla_decode_workload_sampled():
    """256 sequences x 4096 cached tokens x 96 heads, the measured workload,
    compared on sampled sequences."""
    print("mla B=256 L=4096 H=96 (sampled)", flush=True)
    inp = synth.mla_inputs(synth.MLA["decode"], device="cuda")
    y = _run(inp)
    seqs = [0, 255]
    assert report("y (sampled)", f64(y[seqs]), _oracle(inp, seqs=seqs), TOL_BF16) <= TOL_BF16
