"""The parity checker itself (tests/kda_testlib.report), on the CPU: a
correct result passes, and one wrong 16-token chunk fails at the lengths of
the long-context tests, where it moves the whole-tensor rel-L2 by less than
the tolerance.  Synthetic arrays only; no GPU and no oracle."""
import numpy as np
import pytest

from tests.kda_testlib import ELEM, TOL, parity_metrics, report


def _pair(T, H=2, D=None, noise=4e-3, seed=0):
    # (narrower rows at 2^20 tokens keep the arrays small; the chunk count is
    # what matters)
    D = D or (128 if T <= 65536 else 16)
    rng = np.random.default_rng(seed)
    ref = rng.standard_normal((T, H, D))
    gpu = ref * (1 + noise * rng.standard_normal(ref.shape))
    return gpu, ref


@pytest.mark.parametrize("T", [65536, 1 << 20])
def test_correct_result_passes(T):
    gpu, ref = _pair(T)
    assert report("o", gpu, ref, TOL["bf16"]) <= TOL["bf16"]


@pytest.mark.parametrize("T,chunk", [(65536, 1000), (1 << 20, 65535)])
def test_one_wrong_chunk_fails(T, chunk):
    gpu, ref = _pair(T)
    gpu[16 * chunk:16 * chunk + 16] = 0.0     # a chunk whose output was never written
    m = parity_metrics(gpu, ref)
    # the whole-tensor norm alone would pass it
    assert m["rel_l2"] <= TOL["bf16"], m
    assert m["max_block_rel_l2"] > 0.5 and m["worst_block"] == chunk, m
    with pytest.raises(AssertionError):
        report("o", gpu, ref, TOL["bf16"])


def test_twenty_wrong_chunks_at_1M_fail():
    """About 20 wrong chunks still pass a whole-tensor rel-L2 at 2^20 tokens."""
    T = 1 << 20
    gpu, ref = _pair(T, H=1)
    for c in range(0, 65536, 3277):
        gpu[16 * c:16 * c + 16] = 0.0
    assert parity_metrics(gpu, ref)["rel_l2"] <= TOL["bf16"]
    with pytest.raises(AssertionError):
        report("o", gpu, ref, TOL["bf16"])


def test_zeroed_chunk_of_small_values_fails():
    """A chunk whose reference is small (a floor of a quarter of the typical
    block norm applies) still fails when it is zeroed."""
    gpu, ref = _pair(4096)
    ref[160:176] *= 0.3
    gpu[160:176] = 0.0
    with pytest.raises(AssertionError):
        report("o", gpu, ref, TOL["bf16"])


def test_single_wrong_element_fails_elementwise_bar():
    """For the elementwise stages one element off by 1% fails although every
    norm passes."""
    rng = np.random.default_rng(2)
    ref = rng.standard_normal((65536, 2, 128))
    gpu = ref * (1 + 2.0 ** -10 * rng.uniform(-1, 1, ref.shape))    # within the bf16 bound
    assert report("y", gpu, ref, TOL["bf16"], elem=ELEM["bf16"]) <= TOL["bf16"]
    gpu[12345, 1, 7] = ref[12345, 1, 7] * 1.01 + 0.01
    m = parity_metrics(gpu, ref)
    assert m["rel_l2"] <= TOL["bf16"] and m["max_block_rel_l2"] <= TOL["bf16"], m
    with pytest.raises(AssertionError):
        report("y", gpu, ref, TOL["bf16"], elem=ELEM["bf16"])
    with pytest.raises(AssertionError):          # and so does an explicit max-abs bar
        report("y", gpu, ref, TOL["bf16"], max_abs_rms=0.005)


def test_fp32_bar():
    gpu, ref = _pair(256, noise=3e-7)
    assert report("o", gpu, ref, TOL["f32"]) <= TOL["f32"]
    gpu[17] *= 1.001                             # one wrong token
    with pytest.raises(AssertionError):
        report("o", gpu, ref, TOL["f32"])


def test_ragged_tail_block_and_empty():
    gpu, ref = _pair(1000 + 7)
    assert report("o", gpu, ref, TOL["bf16"]) <= TOL["bf16"]
    gpu[-3:] = 0.0
    with pytest.raises(AssertionError):
        report("o", gpu, ref, TOL["bf16"])
    e = np.zeros((0, 2, 4))
    assert report("empty", e, e, TOL["bf16"]) == 0.0


def test_mxfp8_code_window_bounds_an_fp32_evaluation():
    """The per-element error bound that widens the MXFP8 code check's ties
    (tests/test_gpu_mxfp8._error_bound) covers an fp32 evaluation of conv,
    SiLU and L2 against the fp64 oracle, with room to spare, and is not
    vacuous (far below the values themselves)."""
    import torch
    from oracle import c_oracle, kda_ref
    from tests.test_gpu_mxfp8 import _error_bound
    rng = np.random.default_rng(0)
    H, D, N = 3, 128, 300
    P = 3 * H * D
    xs = torch.from_numpy(rng.standard_normal((N, P))).to(torch.bfloat16).double().numpy()
    ws = (rng.standard_normal((P, 4)) * 0.25).astype(np.float32).astype(np.float64)
    ys, _ = c_oracle.short_conv_silu(xs, ws, None)
    u_pre = ys.reshape(N, 3, H, D)
    ref = u_pre.copy()
    ref[:, :2] = kda_ref.l2norm(ref[:, :2])
    err = _error_bound(xs, ws, None, [0, N], u_pre)
    x32, w32 = xs.astype(np.float32), ws.astype(np.float32)
    xp = np.concatenate([np.zeros((3, P), np.float32), x32], 0)
    pre = np.zeros((N, P), np.float32)
    for j in range(4):
        pre = (pre + w32[:, j] * xp[j:j + N]).astype(np.float32)
    u = (pre / (np.float32(1) + np.exp(-pre))).astype(np.float32).reshape(N, 3, H, D)
    ss = np.square(u[:, :2]).sum(-1, keepdims=True, dtype=np.float32)
    y32 = u.copy()
    y32[:, :2] = u[:, :2] * (np.float32(1) / np.sqrt(ss + np.float32(1e-6)))
    assert np.all(np.abs(y32 - ref) <= 0.5 * err)
    assert np.median(err / np.maximum(np.abs(ref), 1e-30)) < 1e-4
