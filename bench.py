"""Benchmark of the KDA token mixer on one MI355X.

A step is one pass of the prefill path over the long-context workload
(B = 1, T = 65,536, 96 heads x 128, bf16 I/O, fp32 state, 16-token chunks):
kda_conv -> kda_chunk_prefill -> kda_gated_norm, inputs resident in HBM.
``value`` is prefill tokens/s.  The decode step (B = 256, 64 consecutive
steps) is timed in the same run and reported as TB/s under ``decode``.

The same run also times the prefill step with MXFP8 activations between
the kernels (E4M3 codes with E8M0 block scales: kda_conv_mxfp8 ->
kda_chunk_prefill_mxfp8 -> kda_gated_norm), the other two
prefill workloads, decode with K tokens per call, the latent-attention decode
step, and the chunk kernel alone over one sequence of 2^20 tokens (the
1M-token regime).

The roofline object describes the dominant kernel (the chunkwise recurrence):
achieved = its algorithmic bytes per launch / its average launch duration,
timed with HIP events on the stream it runs on.  ``cpu_baseline`` times the
CPU oracle on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s + decode TB/s at 96x128 heads; % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_prefill_T65536_traffic.json")
CHUNK_SOURCES = [os.path.join(ROOT, "linear_attention_recurrence_09_amd", "csrc", f)
                 for f in ("kda_chunk_pipe.hip", "kda_chunk.hip", "kda_device.hpp")]
CHUNK_KERNEL = "chunk_pipe_kernel<DK=128, 64 value columns> (kda_chunk_prefill, chunk 16)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def chunk_source_hash():
    """Hash of the chunk-kernel sources without their comments and blank
    lines, so that a change of wording alone keeps the counters current."""
    h = hashlib.sha256()
    for p in CHUNK_SOURCES:
        with open(p, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for line in text.splitlines():
            line = line.split("//", 1)[0].rstrip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per chunk-kernel launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != chunk_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def prefill_bytes(N, H, D, n_seqs, es=2):
    """Algorithmic HBM bytes of each prefill kernel (one launch each)."""
    P = 3 * H * D
    chunk = (4 * N * H * D * es          # q, k, v, g
             + N * H * es                # beta
             + N * H * D * es            # o
             + n_seqs * H * D * D * 4)   # final state (no initial state here)
    conv = 2 * N * P * es               # x in, y out
    norm = 3 * N * H * D * es           # o, gate in, y out
    return dict(conv=conv, chunk=chunk, norm=norm)


def mxfp8_chunk_bytes(N, H, D, n_seqs):
    """Algorithmic HBM bytes of one kda_chunk_prefill_mxfp8 launch: q, k, v, g
    as one-byte codes plus one scale byte per 32 values, beta and o in bf16,
    the final state in fp32."""
    return (4 * N * H * D              # q, k, v, g codes
            + 4 * N * H * (D // 32)    # their block scales
            + N * H * 2                # beta
            + N * H * D * 2            # o
            + n_seqs * H * D * D * 4)  # final state


def chunk_flops(N, H, D, C=16):
    """Algorithmic FLOPs of the chunked recurrence, triangular-exact: per chunk
    A_kk (strictly lower) and A_qk (lower) over D channels, the unit triangular
    inverse (C^3/3), U = M'(V - K~S), O = Q~S + A_qk U and the state update."""
    per_chunk = (C * (C - 1) * D          # A_kk
                 + C * (C + 1) * D        # A_qk
                 + C ** 3 / 3             # inverse
                 + 2 * C * D * D          # K~ S
                 + C * (C + 1) * D        # M' Z
                 + 2 * C * D * D          # Q~ S
                 + C * (C + 1) * D        # A_qk U
                 + 2 * C * D * D)         # K^^T U
    return per_chunk / C * N * H


def decode_bytes(B, H, D, es=2):
    P = 3 * H * D
    return (2 * B * H * D * D * 4        # state read + write
            + 2 * B * P * 3 * es         # rolling conv state read + write
            + B * P * es                 # new token x
            + B * H * D * es             # g
            + B * H * es                 # beta
            + B * H * D * es             # o
            + P * 4 * 4)                 # conv weights


def decode_multi_bytes(B, K, H, D, es=2, write_states=True, outputs=True):
    """Algorithmic HBM bytes of one kda_decode_multi call of K tokens."""
    P = 3 * H * D
    states = B * H * D * D * 4 + B * P * 3 * es
    return ((2 if write_states else 1) * states
            + B * K * (P * es + H * D * es + H * es)   # x, g, beta
            + (B * K * H * D * es if outputs else 0)   # o
            + P * 4 * 4)                               # conv weights


def mla_bytes(B, H, L, R=512, Dh=128, es=2):
    """Algorithmic HBM bytes of one latent-attention decode step: the cached
    latents once, both up-projections, the query, gate and output (the split
    partials in the workspace are the kernel's own, not counted)."""
    return B * L * R * es + 2 * H * Dh * R * es + 3 * B * H * Dh * es


def mla_flops(B, H, L, R=512, Dh=128):
    """Scores q'.c and the weighted latent sum (2 R each per head and cached
    token), plus the two per-head projections q' = W_uk^T q and o = W_uv u."""
    return B * H * (4 * L * R + 4 * Dh * R)


def bench_mla(kda, synth, torch, stream, reps, block=5):
    """One latent-attention decode step over a 4096-token latent cache for
    256 sequences and 96 heads, timed with HIP events on the launch stream:
    steps issued back to back in blocks of `block` (one event pair per block,
    so the events and the host's launch gaps do not sit between the steps, as
    in a decode loop where the layers run one after another), reported per
    step; the median over `reps` blocks."""
    spec = synth.MLA["decode"]
    B, H, L = spec.B, spec.H, spec.L_max
    log(f"drawing inputs for {spec.name}")
    inp = synth.mla_inputs(spec, device="cuda")
    y = torch.empty((B, H, spec.Dh), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(kda.kda_mla_decode_workspace_bytes(B, H, L), dtype=torch.uint8,
                     device="cuda")

    def call():
        kda.kda_mla_decode(inp["q"], inp["w_uk"], inp["w_uv"], inp["cache"], inp["lengths"],
                           inp["gate"], y, B, H, L, workspace=ws, stream=stream)

    for _ in range(3):
        call()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record(stream)
        for _ in range(block):
            call()
        e1.record(stream)
    torch.cuda.synchronize()
    per = sorted(e0.elapsed_time(e1) / block for e0, e1 in evs)
    med = per[len(per) // 2]
    nb, fl = mla_bytes(B, H, L), mla_flops(B, H, L)
    log(f"mla decode: {med:.3f} ms/step, {nb / med / 1e9:.2f} TB/s")
    del inp, y, ws
    return {"workload": spec.name, "B": B, "H": H, "L": L, "R": spec.R,
            "timing": f"median over {reps} blocks of {block} steps issued back to back",
            "ms_per_step_median": med, "ms_per_step_min": per[0], "ms_per_step_max": per[-1],
            "bytes_per_step": nb, "TBps": nb / (med * 1e-3) / 1e12,
            "hbm_frac": nb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "tflops_algorithmic": fl / (med * 1e-3) / 1e12,
            "mfma_frac": fl / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "tokens_per_s": B / (med * 1e-3)}


def bench_chunk_1m(kda, torch, stream, H, D, C, steps):
    """kda_chunk_prefill on one sequence of 2^20 tokens: q and k with unit
    norm on average, v in [-1, 1], log-decay in [-5, 0], beta in (0.1, 0.9)."""
    N = 1 << 20
    HD = H * D
    log(f"allocating the 1M-token chunk workload ({N} tokens, {H} heads)")
    y_qkv = torch.empty((N, 3 * HD), dtype=torch.bfloat16, device="cuda")
    y_qkv[:, :2 * HD].uniform_(-0.15, 0.15)
    y_qkv[:, 2 * HD:].uniform_(-1.0, 1.0)
    g = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda").uniform_(-5.0, 0.0)
    beta = torch.empty((N, H), dtype=torch.bfloat16, device="cuda").uniform_(0.1, 0.9)
    o = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda")
    sT = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")

    def call():
        kda.kda_chunk_prefill(y_qkv[:, :HD], y_qkv[:, HD:2 * HD], y_qkv[:, 2 * HD:], 3 * HD, g,
                              beta, o, 1, N, H, D, D, chunk=C, final_state=sT, stream=stream)

    call()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps
    finite = bool(torch.isfinite(sT).all())
    nb = prefill_bytes(N, H, D, 1)["chunk"]
    log(f"1M-token chunk kernel: {ms:.2f} ms, {N / ms / 1e3:.2f} M tokens/s")
    del y_qkv, g, beta, o, sT
    torch.cuda.empty_cache()
    return {"workload": f"chunk_prefill_T{N}_H{H}_D{D}_bf16 (one sequence)", "tokens": N,
            "steps": steps, "ms_per_call": ms, "tokens_per_s": N / (ms * 1e-3),
            "achieved_GBs": nb / (ms * 1e-3) / 1e9,
            "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "final_state_finite": finite}


def mxfp8_conv_bytes(N, H, D):
    """Algorithmic HBM bytes of one kda_conv_mxfp8 launch: bf16 x in, one
    code byte per channel and one scale byte per 32 channels out."""
    P = 3 * H * D
    return 2 * N * P + N * P + N * P // 32


def bench_mxfp8_prefill(kda, synth, torch, stream, x, w, g, beta, gate, nw, H, D, steps, warmup):
    """The prefill step with MXFP8 activations between the kernels:
    kda_conv_mxfp8 -> kda_chunk_prefill_mxfp8 -> kda_gated_norm, on the same
    inputs as the bf16 step; g is encoded to MXFP8 outside the timed region
    (its producer is outside this path).  HIP events on the launch stream."""
    N, HD = x.shape[0], H * D
    P = 3 * HD
    codes = torch.empty((N, P), dtype=torch.uint8, device="cuda")
    sc = [torch.empty((N, H, D // 32), dtype=torch.uint8, device="cuda") for _ in range(3)]
    gc, gs = synth.mxfp8_encode(g)
    gc, gs = gc.contiguous(), gs.contiguous()
    o = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(o)
    sT = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        kda.kda_conv_mxfp8(x, w, codes, *sc, 1, N, H, D, stream=stream)
        if ev:
            ev[1].record(stream)
        kda.kda_chunk_prefill_mxfp8(codes[:, :HD], sc[0], codes[:, HD:2 * HD], sc[1],
                                    codes[:, 2 * HD:], sc[2], P, gc, gs, beta, o, 1, N, H,
                                    final_state=sT, stream=stream)
        if ev:
            ev[2].record(stream)
        kda.kda_gated_norm(o, gate, nw, y, N, H, D, stream=stream)
        if ev:
            ev[3].record(stream)

    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    km = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps
          for j, n in enumerate(("conv", "chunk", "norm"))}
    nb = {"conv": mxfp8_conv_bytes(N, H, D), "chunk": mxfp8_chunk_bytes(N, H, D, 1),
          "norm": prefill_bytes(N, H, D, 1)["norm"]}
    log(f"MXFP8 prefill: {ms_step:.3f} ms/step ({N / ms_step / 1e3:.2f} M tokens/s); "
        f"kernels {km}")
    del codes, sc, gc, gs, o, y, sT
    return {"workload": f"prefill_T{N}_H{H}_D{D}_mxfp8: kda_conv_mxfp8 -> "
                        f"kda_chunk_prefill_mxfp8 -> kda_gated_norm (q, k, v, g as E4M3 codes "
                        f"with one E8M0 scale per 32 values; x, beta, gate, o, y bf16)",
            "tokens": N, "steps": steps, "ms_per_step": ms_step,
            "tokens_per_s": N / (ms_step * 1e-3), "kernels_ms": km,
            "bytes_per_launch": nb,
            "kernels_GBs": {k: nb[k] / (km[k] * 1e-3) / 1e9 for k in km},
            "kernels_hbm_frac": {k: nb[k] / (km[k] * 1e-3) / 1e9 / HBM_PEAK_GBS for k in km}}


def _cpu_info():
    """Host CPU model, nominal clock and the threads this process may use."""
    model, mhz = "unknown", None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name") and model == "unknown":
                    model = line.split(":", 1)[1].strip()
                elif line.startswith("cpu MHz") and mhz is None:
                    mhz = float(line.split(":", 1)[1])
    except (OSError, ValueError):
        pass
    return {"cpu_model": model, "cpu_mhz": mhz, "affinity_cores": len(os.sched_getaffinity(0))}


def parity_figures(gpu, ref, block=16):
    """rel-L2, the largest rel-L2 over blocks of `block` rows of the leading
    (token) axis, max-abs and max-abs over the reference's RMS."""
    import numpy as np
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    d = g - r
    rn = float(np.linalg.norm(r))
    rms = rn / np.sqrt(r.size)
    rows = r.shape[0]
    nb = rows // block
    worst = 0.0
    if nb:
        bd = np.sqrt(np.square(d[:nb * block]).reshape(nb, -1).sum(axis=1))
        br = np.sqrt(np.square(r[:nb * block]).reshape(nb, -1).sum(axis=1))
        floor = 0.25 * rms * np.sqrt(r[:block].size)
        worst = float((bd / np.maximum(br, floor)).max())
    ma = float(np.abs(d).max())
    return {"rel_l2": float(np.linalg.norm(d) / rn), "max_block_rel_l2": worst,
            "max_abs": ma, "max_abs_over_rms": ma / rms}


def bench_fused_prefill(kda, torch, stream, x, w, g, beta, gate, nw, H, D, steps, warmup):
    """kda_prefill_fused on the same inputs as the three-call step: the conv,
    SiLU and L2 inside the recurrence kernel, then the gated norm (y written
    over o).  HIP events on the launch stream; the fused floor is the bytes a
    single pass would move (x, g, beta, gate in, y out), this path's bytes
    add the recurrence's o out and back in."""
    N = x.shape[0]
    o = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda")
    sT = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")

    def step():
        kda.kda_prefill_fused(x, w, g, beta, gate, nw, o, o, H, D, B=1, T=N, final_state=sT,
                              stream=stream)

    for _ in range(warmup):
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    per = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    ms = sum(per) / steps
    P = 3 * H * D
    floor_b = N * P * 2 + 2 * N * H * D * 2 + N * H * 2 + N * H * D * 2      # x, g, gate, beta, y
    path_b = floor_b + 2 * N * H * D * 2                                     # + o out and in
    log(f"fused prefill: {ms:.3f} ms/step ({N / ms / 1e3:.2f} M tokens/s)")
    del o, sT
    return {"workload": f"prefill_T{N}_H{H}_D{D}_bf16 through kda_prefill_fused (conv + SiLU + L2 "
                        f"inside the recurrence kernel, then the gated norm)",
            "tokens": N, "steps": steps, "ms_per_step": ms,
            "ms_median_min_max": [per[len(per) // 2], per[0], per[-1]],
            "tokens_per_s": N / (ms * 1e-3),
            "fused_floor_bytes": floor_b, "fused_floor_ms": floor_b / HBM_PEAK_GBS / 1e6,
            "path_bytes": path_b, "path_floor_ms": path_b / HBM_PEAK_GBS / 1e6,
            "hbm_frac_of_fused_floor": floor_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def cpu_baseline(inp, spec, T_s, H_s, gpu_out):
    """The CPU oracle on the first T_s tokens of the first H_s heads (all its
    threads), plus one-thread figures on the tiny workload and on a sample of
    the T = 4,096 workload; and the parity of the timed GPU step's outputs
    (o, y, final state) on the same heads against that oracle run."""
    import torch
    import synth
    from oracle import c_oracle
    nthr = c_oracle.num_threads()
    H_s = min(H_s, spec.H)
    heads = list(range(H_s))
    H, D = spec.H, spec.D
    cols = []
    for part in range(3):
        for h in heads:
            cols.extend(range(part * H * D + h * D, part * H * D + (h + 1) * D))
    cols_t = torch.as_tensor(cols, device=inp["x"].device)
    f = lambda t: t.detach().double().cpu().numpy()
    xs = f(inp["x"][:T_s].index_select(1, cols_t))
    ws = f(inp["conv_w"].index_select(0, cols_t))
    gs, bs, zs = f(inp["g"][:T_s, heads]), f(inp["beta"][:T_s, heads]), f(inp["gate"][:T_s, heads])
    nw = f(inp["norm_w"])
    t0 = time.perf_counter()
    ref = c_oracle.kda_prefill(xs, ws, gs, bs, zs, nw, [0, T_s], H_s, D)
    dt = time.perf_counter() - t0
    del xs, gs, bs, zs
    parity = {"workload": f"the timed step's outputs, heads 0..{H_s - 1} of {H}, tokens 0.."
                          f"{T_s - 1}, against the C fp64 oracle (bar: 2e-2 for rel-L2 and "
                          f"for every 16-token block)"}
    for key in ("o", "y"):
        parity[key] = parity_figures(f(gpu_out[key][:T_s, heads]), ref[key])
    if T_s == gpu_out["o"].shape[0]:
        parity["S_final"] = parity_figures(f(gpu_out["S_final"][:, heads]), ref["S_final"])
    del ref
    # one host thread: the tiny workload whole, and 2 heads of T = 4,096
    one = {}
    c_oracle.set_num_threads(1)
    try:
        for cid, nh in ((0, None), (1, 2)):
            es = synth.CONFIGS[cid]
            ei = synth.prefill_inputs(es, device="cpu")
            hs = list(range(es.H if nh is None else nh))
            cc = []
            for part in range(3):
                for h in hs:
                    cc.extend(range(part * es.H * es.D + h * es.D, part * es.H * es.D + (h + 1) * es.D))
            cc = torch.as_tensor(cc)
            a = [f(ei["x"].index_select(1, cc)), f(ei["conv_w"].index_select(0, cc)),
                 f(ei["g"][:, hs]), f(ei["beta"][:, hs]), f(ei["gate"][:, hs]), f(ei["norm_w"])]
            t1 = time.perf_counter()
            c_oracle.kda_prefill(*a, ei["cu"], len(hs), es.D)
            d1 = time.perf_counter() - t1
            Ne = ei["x"].shape[0]
            one[es.name] = {"seconds": d1, "heads_run": len(hs), "heads": es.H,
                            "tokens_per_s": Ne * len(hs) / es.H / d1, "cores": 1}
    finally:
        c_oracle.set_num_threads(nthr)
    base = {"value": T_s * H_s / H / dt, "unit": "tokens/s", "cores": min(nthr, H_s),
            "kind": "oracle", **_cpu_info(), "head_scale": H_s / H,
            "sample": (f"C fp64 oracle, whole prefill path (conv, L2, recurrence, gated norm) on "
                       f"the first {T_s} tokens of {H_s} of the {H} heads, {dt:.1f} s on "
                       f"{min(nthr, H_s)} threads; value = tokens/s of the {H}-head layer "
                       f"= {T_s} x {H_s}/{H} / {dt:.1f} s"),
            "one_thread": one}
    return base, parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--cpu-tokens", type=int, default=65536)
    ap.add_argument("--cpu-heads", type=int, default=48)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="short run for rocprofv3 counter passes: each kernel a few times "
                         "(conv, chunk, norm at T=65536; decode at B=256) plus a plain copy "
                         "kernel of known size for calibration")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the KDA mixer here is a single-GPU library "
              f"(requested --gpus {args.gpus}). Across GPUs the heads would be split (each "
              f"rank owns whole heads and their states), which needs no collective inside "
              f"the mixer.", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import linear_attention_recurrence_09_amd as kda
    import synth

    torch.cuda.set_device(0)
    kda.lib()
    spec = synth.CONFIGS[2]
    H, D = spec.H, spec.D
    C = spec.chunk or 16        # 0 selects the library's fastest variant: 16 for bf16
    HD = H * D
    log(f"drawing inputs for {spec.name}")
    inp = synth.prefill_inputs(spec, device="cuda")
    N = inp["x"].shape[0]
    x, w, g, beta, gate, nw = (inp[k] for k in ("x", "conv_w", "g", "beta", "gate", "norm_w"))
    y_qkv = torch.empty_like(x)
    o = torch.empty((N, H, D), dtype=x.dtype, device="cuda")
    y = torch.empty_like(o)
    sT = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
          for _ in range(args.steps)]

    def step(events=None):
        if events:
            events[0].record(stream)
        kda.kda_conv(x, w, y_qkv, 1, N, H, D, stream=stream)
        if events:
            events[1].record(stream)
        kda.kda_chunk_prefill(y_qkv[:, :HD], y_qkv[:, HD:2 * HD], y_qkv[:, 2 * HD:], 3 * HD, g,
                              beta, o, 1, N, H, D, D, chunk=C, final_state=sT, stream=stream)
        if events:
            events[2].record(stream)
        kda.kda_gated_norm(o, gate, nw, y, N, H, D, stream=stream)
        if events:
            events[3].record(stream)

    if args.counters:
        # the recurrence kernel alone (after one conv pass to produce its
        # inputs), then an elementwise copy of 2 GiB in and 2 GiB out, whose
        # byte counters calibrate the recurrence's
        kda.kda_conv(x, w, y_qkv, 1, N, H, D, stream=stream)
        for _ in range(3):
            kda.kda_chunk_prefill(y_qkv[:, :HD], y_qkv[:, HD:2 * HD], y_qkv[:, 2 * HD:], 3 * HD,
                                  g, beta, o, 1, N, H, D, D, chunk=C, final_state=sT,
                                  stream=stream)
        kda.kda_gated_norm(o, gate, nw, y, N, H, D, stream=stream)
        # the MXFP8 step on the same inputs, three times (conv, chunk, norm)
        bench_mxfp8_prefill(kda, synth, torch, stream, x, w, g, beta, gate, nw, H, D, steps=3,
                            warmup=0)
        # the fused prefill on the same inputs, three times
        bench_fused_prefill(kda, torch, stream, x, w, g, beta, gate, nw, H, D, steps=3, warmup=0)
        # the decode kernels: three one-token steps, two calls of four tokens
        dspec = synth.CONFIGS[4]
        Bd, Hd, Dd = dspec.B, dspec.H, dspec.D
        d = synth.decode_inputs(dspec, device="cuda", steps=4)
        od = torch.empty((Bd, Hd, Dd), dtype=d["x"].dtype, device="cuda")
        cs, S = d["conv_state"].clone(), d["S0"].clone()
        for t in range(3):
            kda.kda_decode_step(d["x"][t], d["conv_w"], cs, d["g"][t], d["beta"][t], S, od, Bd,
                                Hd, Dd, stream=stream)
        xb, gb, bb = (d[n].transpose(0, 1).contiguous() for n in ("x", "g", "beta"))
        om = torch.empty((Bd, 4, Hd, Dd), dtype=d["x"].dtype, device="cuda")
        for _ in range(2):
            kda.kda_decode_multi(xb, d["conv_w"], cs, gb, bb, S, Bd, 4, Hd, Dd, o=om,
                                 conv_state_out=cs, state_out=S, stream=stream)
        torch.cuda.synchronize()
        del d, cs, S, xb, gb, bb, om
        # six latent-attention decode steps (256 x 4096 cached latents)
        bench_mla(kda, synth, torch, stream, reps=1, block=3)
        src = torch.empty(1 << 29, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log("counter run done: conv, 3 chunk launches, norm, 3 MXFP8 prefill steps, 3 fused "
            "prefill steps, 3 decode "
            "steps, 2 four-token decode calls, 6 latent-attention decode steps, 3 copies of "
            "2 GiB")
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    k_ms = {"conv": 0.0, "chunk": 0.0, "norm": 0.0}
    for e in ev:
        k_ms["conv"] += e[0].elapsed_time(e[1]) / args.steps
        k_ms["chunk"] += e[1].elapsed_time(e[2]) / args.steps
        k_ms["norm"] += e[2].elapsed_time(e[3]) / args.steps
    chunk_each = sorted(e[1].elapsed_time(e[2]) for e in ev)
    log(f"timed prefill: {ms_step:.3f} ms/step; kernels {k_ms}")

    nbytes = prefill_bytes(N, H, D, 1)
    achieved = nbytes["chunk"] / (k_ms["chunk"] * 1e-3) / 1e9
    flops = chunk_flops(N, H, D, C)
    traffic = measured_traffic()
    result = {
        "metric": METRIC,
        "value": N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded device-drawn inputs with the pages' layer shape and value "
                "distributions (no dataset or weights involved)",
        "config": {"workload": "prefill_T65536_H96_D128_bf16: conv+SiLU+L2 -> chunked gated "
                               "delta rule -> gated RMSNorm",
                   "T": N, "H": H, "D": D, "chunk": C, "sequences": 1, "state": "fp32"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": CHUNK_KERNEL,
                     "algorithmic_bytes_per_launch": nbytes["chunk"],
                     "avg_launch_ms": k_ms["chunk"],
                     "launch_ms_median_min_max": [chunk_each[len(chunk_each) // 2],
                                                  chunk_each[0], chunk_each[-1]],
                     "mfma_tflops_algorithmic": flops / (k_ms["chunk"] * 1e-3) / 1e12,
                     "mfma_frac": flops / (k_ms["chunk"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "kernels_ms": k_ms,
        "pipeline_gbs": sum(nbytes.values()) / (ms_step * 1e-3) / 1e9,
    }

    result["prefill_T65536_fused"] = bench_fused_prefill(
        kda, torch, stream, x, w, g, beta, gate, nw, H, D, args.steps, args.warmup)

    result["prefill_T65536_mxfp8"] = bench_mxfp8_prefill(
        kda, synth, torch, stream, x, w, g, beta, gate, nw, H, D, args.steps, args.warmup)

    # the other two prefill workloads, timed the same way (informative: the
    # headline value is the workload above)
    extra = {}
    flush = torch.empty(1 << 27, dtype=torch.float32, device="cuda")
    for cid in (1, 3):
        es = synth.CONFIGS[cid]
        ei = synth.prefill_inputs(es, device="cuda")
        Ne, Se = ei["x"].shape[0], len(ei["lengths"])
        cu = (torch.tensor(ei["cu"], dtype=torch.int32, device="cuda") if es.varlen else None)
        ye = torch.empty_like(ei["x"])
        oe = torch.empty((Ne, H, D), dtype=ei["x"].dtype, device="cuda")
        yn = torch.empty_like(oe)
        sTe = torch.empty((Se, H, D, D), dtype=torch.float32, device="cuda")
        Be, Te = (1, Ne) if es.varlen else (Se, Ne // Se)

        def estep(events=None):
            if events:
                events[0].record(stream)
            kda.kda_conv(ei["x"], ei["conv_w"], ye, Be, Te, H, D, cu_seqlens=cu, num_seqs=Se,
                         stream=stream)
            if events:
                events[1].record(stream)
            kda.kda_chunk_prefill(ye[:, :HD], ye[:, HD:2 * HD], ye[:, 2 * HD:], 3 * HD, ei["g"],
                                  ei["beta"], oe, Be, Te, H, D, D, chunk=C,
                                  initial_state=ei["S0"], final_state=sTe, cu_seqlens=cu,
                                  num_seqs=Se, stream=stream)
            if events:
                events[2].record(stream)
            kda.kda_gated_norm(oe, ei["gate"], ei["norm_w"], yn, Ne, H, D, stream=stream)
            if events:
                events[3].record(stream)

        for _ in range(args.warmup):
            estep()
        eev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            flush.fill_(float(i))      # 512 MB written between repetitions (caches flushed)
            estep(eev[i])
        torch.cuda.synchronize()
        km = {n: sum(e[j].elapsed_time(e[j + 1]) for e in eev) / args.steps
              for j, n in enumerate(("conv", "chunk", "norm"))}
        ms = sum(km.values())
        extra[es.name] = {"tokens": Ne, "sequences": Se, "ms_per_step": ms,
                          "tokens_per_s": Ne / (ms * 1e-3), "kernels_ms": km,
                          "timing": "kernel events; a 512 MB buffer written before each step"}
        log(f"{es.name}: {ms:.3f} ms/step, {Ne / ms / 1e3:.2f} M tokens/s")
        del ei, ye, oe, yn, sTe
    result["prefill_other_workloads"] = extra
    del flush

    if not args.no_decode:
        dspec = synth.CONFIGS[4]
        B, Hd, Dd = dspec.B, dspec.H, dspec.D
        steps = args.decode_steps
        log(f"drawing inputs for {dspec.name}")
        d = synth.decode_inputs(dspec, device="cuda", steps=steps)
        od = torch.empty((B, Hd, Dd), dtype=d["x"].dtype, device="cuda")

        def decode_pass(cs, S, events=None):
            for t in range(steps):
                if events:
                    events[t][0].record(stream)
                kda.kda_decode_step(d["x"][t], d["conv_w"], cs, d["g"][t], d["beta"][t], S, od,
                                    B, Hd, Dd, stream=stream)
                if events:
                    events[t][1].record(stream)

        decode_pass(d["conv_state"].clone(), d["S0"].clone())    # warm-up on copies
        torch.cuda.synchronize()
        dev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        cs, S = d["conv_state"].clone(), d["S0"].clone()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        decode_pass(cs, S, dev)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        per = sorted(e[0].elapsed_time(e[1]) for e in dev)
        med = per[len(per) // 2]
        db = decode_bytes(B, Hd, Dd)
        result["decode"] = {"workload": dspec.name, "B": B, "steps": steps,
                            "ms_per_step_median": med, "ms_per_step_min": per[0],
                            "ms_per_step_max": per[-1],
                            "wall_ms_per_step": (t1 - t0) * 1e3 / steps,
                            "bytes_per_step": db, "TBps": db / (med * 1e-3) / 1e12,
                            "tokens_per_s": B / (med * 1e-3),
                            "hbm_frac": db / (med * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log(f"decode: {med:.3f} ms/step, {result['decode']['TBps']:.2f} TB/s")

        # K tokens per call (checking drafted tokens): the same 64 tokens per
        # sequence as 64 / K calls, states in place, every token accepted
        per_k = {}
        for K in (2, 4, 8):
            calls = steps // K
            blk = [(d["x"][c * K:(c + 1) * K].transpose(0, 1).contiguous(),
                    d["g"][c * K:(c + 1) * K].transpose(0, 1).contiguous(),
                    d["beta"][c * K:(c + 1) * K].transpose(0, 1).contiguous())
                   for c in range(calls)]
            om = torch.empty((B, K, Hd, Dd), dtype=d["x"].dtype, device="cuda")

            def multi_pass(cs, S, events=None):
                for c, (xb, gb, bb) in enumerate(blk):
                    if events:
                        events[c][0].record(stream)
                    kda.kda_decode_multi(xb, d["conv_w"], cs, gb, bb, S, B, K, Hd, Dd, o=om,
                                         conv_state_out=cs, state_out=S, stream=stream)
                    if events:
                        events[c][1].record(stream)

            multi_pass(d["conv_state"].clone(), d["S0"].clone())
            cs, S = d["conv_state"].clone(), d["S0"].clone()
            mev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(calls)]
            torch.cuda.synchronize()
            multi_pass(cs, S, mev)
            torch.cuda.synchronize()
            per = sorted(e[0].elapsed_time(e[1]) for e in mev)
            med = per[len(per) // 2]
            mb = decode_multi_bytes(B, K, Hd, Dd)
            per_k[str(K)] = {"calls": calls, "ms_per_call_median": med, "ms_per_call_min": per[0],
                             "ms_per_call_max": per[-1], "bytes_per_call": mb,
                             "TBps": mb / (med * 1e-3) / 1e12,
                             "tokens_per_s": B * K / (med * 1e-3),
                             "hbm_frac": mb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS}
            log(f"decode_multi K={K}: {med:.3f} ms/call, {B * K / med:.0f}k tokens/s")
            del blk, om
        # the check-then-accept pair at K = 4: outputs only, then the accepted
        # tokens (all four, the most state work) in place
        K = 4
        xb, gb, bb = (d[n][:K].transpose(0, 1).contiguous() for n in ("x", "g", "beta"))
        om = torch.empty((B, K, Hd, Dd), dtype=d["x"].dtype, device="cuda")
        acc = torch.full((B,), K, dtype=torch.int32, device="cuda")
        cs, S = d["conv_state"].clone(), d["S0"].clone()
        pair_ms = []
        for rep in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            kda.kda_decode_multi(xb, d["conv_w"], cs, gb, bb, S, B, K, Hd, Dd, o=om, stream=stream)
            kda.kda_decode_multi(xb, d["conv_w"], cs, gb, bb, S, B, K, Hd, Dd, conv_state_out=cs,
                                 state_out=S, n_tokens=acc, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            if rep:
                pair_ms.append(e0.elapsed_time(e1))
        pair_ms.sort()
        pmed = pair_ms[len(pair_ms) // 2]
        result["decode_multi"] = {
            "workload": f"{dspec.name}: K tokens per call, states in place",
            "B": B, "per_K": per_k,
            "check_then_accept_K4": {
                "ms_median": pmed, "tokens_per_s": B * K / (pmed * 1e-3),
                "bytes": decode_multi_bytes(B, K, Hd, Dd, write_states=False)
                         + decode_multi_bytes(B, K, Hd, Dd, outputs=False)}}
        del d, cs, S

    if not args.no_decode:
        result["mla_decode"] = bench_mla(kda, synth, torch, stream, reps=max(args.steps, 10))


    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        result["cpu_baseline"], result["parity"] = cpu_baseline(
            inp, spec, args.cpu_tokens, args.cpu_heads, {"o": o, "y": y, "S_final": sT})
        log(f"cpu baseline: {result['cpu_baseline']['value']:.1f} tokens/s; parity "
            f"{json.dumps(result['parity'])}")
    # the 1M-token regime: the chunk kernel alone over one sequence of
    # 1,048,576 tokens at 96 x 128 (129 GB of device buffers, filled in place
    # in bf16 with the value ranges of the workloads above)
    del inp, x, w, g, beta, gate, nw, y_qkv, o, y
    torch.cuda.empty_cache()
    result["prefill_T1048576_chunk"] = bench_chunk_1m(kda, torch, stream, H, D, C,
                                                      steps=max(args.steps // 3, 3))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
