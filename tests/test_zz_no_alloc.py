"""kda_mla_decode_noalloc, the latent-attention decode entry point that
allocates nothing (its scratch is a static device array of the library),
against kda_mla_decode with a caller-owned workspace: two calls in a row on
the same GPU, the second with a smaller input, each bitwise equal to the
workspace entry point's result on the same inputs (the same kernels run),
and the first also against the oracle.  A request beyond the static scratch
is refused before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import linear_attention_recurrence_09_amd as kda
import synth
from oracle import kda_ref
from tests.kda_testlib import f64, report

pytestmark = pytest.mark.gpu


def _both(spec, lengths):
    inp = synth.mla_inputs(spec, device="cuda", lengths=lengths)
    B, H, L = spec.B, spec.H, spec.L_max
    y_ws = torch.empty((B, H, spec.Dh), dtype=torch.bfloat16, device="cuda")
    y_na = torch.full_like(y_ws, float("nan"))
    ws = torch.empty(kda.kda_mla_decode_workspace_bytes(B, H, L), dtype=torch.uint8,
                     device="cuda")
    args = (inp["q"], inp["w_uk"], inp["w_uv"], inp["cache"], inp["lengths"], inp["gate"])
    kda.kda_mla_decode(*args, y_ws, B, H, L, workspace=ws)
    kda.kda_mla_decode_noalloc(*args, y_na, B, H, L)
    torch.cuda.synchronize()
    return inp, y_ws, y_na


def test_noalloc_matches_workspace_entry_point_twice():
    big = synth.MlaSpec("mla_B64_L1024_H96", B=64, H=96, L_max=1024, seed=3101)
    small = synth.MlaSpec("mla_B8_L200_H32", B=8, H=32, L_max=200, seed=3102)
    print("first call: B=64, H=96, L_max=1024 (ragged lengths)", flush=True)
    inp, y_ws, y_na = _both(big, [1 + (37 * b) % 1024 for b in range(64)])
    assert torch.equal(y_na, y_ws), "first call differs from kda_mla_decode"
    seqs = [0, 17, 63]
    idx = torch.tensor(seqs, device="cuda")
    q, cache, gate = (inp[k].index_select(0, idx) for k in ("q", "cache", "gate"))
    ref = kda_ref.mla_decode(f64(q), f64(inp["w_uk"]), f64(inp["w_uv"]), f64(cache),
                             np.asarray([inp["lengths_list"][b] for b in seqs]), f64(gate))
    report("y (sampled sequences)", f64(y_na[seqs]), ref, 2e-2)
    print("second call: B=8, H=32, L_max=200", flush=True)
    _, y_ws2, y_na2 = _both(small, [200, 1, 33, 150, 64, 65, 2, 199])
    assert torch.equal(y_na2, y_ws2), "second call differs from kda_mla_decode"


def test_noalloc_refuses_beyond_its_scratch():
    """B = 4096 at H = 96 needs about 1.2 GB: refused on the host, nothing
    launched, y untouched."""
    L = kda.lib()
    B, H, Lmax = 4096, 96, 64
    need = kda.kda_mla_decode_workspace_bytes(B, H, Lmax)
    assert need > kda.KDA_MLA_NOALLOC_MAX_BYTES
    dev = lambda n, dt=torch.bfloat16: torch.zeros(n, dtype=dt, device="cuda")
    q, wk, wv = dev(B * H * 128), dev(H * 128 * 512), dev(H * 128 * 512)
    cache, gate = dev(B * Lmax * 512), dev(B * H * 128)
    lengths = torch.ones(B, dtype=torch.int32, device="cuda")
    y = torch.full((B * H * 128,), 7.0, dtype=torch.bfloat16, device="cuda")
    rc = L.kda_mla_decode_noalloc(q.data_ptr(), wk.data_ptr(), wv.data_ptr(), cache.data_ptr(),
                                  lengths.data_ptr(), gate.data_ptr(), y.data_ptr(), B, H, Lmax,
                                  512, 128, 128, ctypes.c_float(128 ** -0.5), kda.KDA_BF16,
                                  None)
    torch.cuda.synchronize()
    assert rc == 1, rc
    assert "static scratch" in kda.kda_last_error()
    assert torch.all(y == 7.0)
