"""Summarise rocprofv3 output of bench.py into profiles/.

Inputs (CSV files written by the commands recorded in the summaries):
  --trace  <dir>/bench_kernel_stats.csv   from
           rocprofv3 --kernel-trace --stats -T -f csv -d <dir> -o bench -- \
               python3 bench.py --steps 20 --warmup 10 --no-cpu-baseline
           (the per-dispatch <dir>/bench_kernel_trace.csv beside it gives the
           average over the 20 timed steps of the headline workload)
  --fetch  <dir>/fetch_counter_collection.csv from
           rocprofv3 --pmc FETCH_SIZE -T -f csv -d <dir> -o fetch -- python3 bench.py --counters
  --write  <dir>/write_counter_collection.csv from
           rocprofv3 --pmc WRITE_SIZE -T -f csv -d <dir> -o write -- python3 bench.py --counters

Writes profiles/chunk_prefill_T65536_kernel_stats.txt (every kernel of the
run, the latent-attention decode kernels included),
profiles/chunk_prefill_T65536_traffic.json and, for every kernel of the
counter run, profiles/kernels_traffic_T65536_B256.txt.  With --l2a/--l2b/--l2c
(three L1/L2 counter passes, L2_PASSES) it writes the memory-path comparison of
the streaming kernels, profiles/memory_path_T65536.txt.  The byte counters (KiB per
dispatch) are scaled by what the same counter reads for bench.py's copy
kernel of known size (2 GiB read, 2 GiB written); the JSON records the hash
of the chunk-kernel sources so bench.py can tell whether it is current.
"""
import argparse
import csv
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

COPY_BYTES = 2 * 1024 ** 3
# mangled names as rocprofv3 -T prints them: the bf16, MXFP8 and fused-conv
# instantiations of the 16-token chunk kernel (input-mode template argument
# 0 / 1 / 2; the bool after it is the output staging, on for one sequence of
# bf16 inputs)
CHUNK_TAG = "chunk_pipe_kernelILi128ELi64ELi0ELb1E"
MX_TAG = "chunk_pipe_kernelILi128ELi64ELi1ELb0E"
CV_TAG = "chunk_pipe_kernelILi128ELi64ELi2ELb0E"
COPY_TAG = "vectorized_elementwise_kernel"


def per_dispatch(path, counter):
    vals = {}
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = r["Dispatch_Id"]
        vals[d] = vals.get(d, 0.0) + float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    return [(names[d], vals[d]) for d in sorted(vals, key=int)]


PMC_PASSES = [
    "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_MFMA SQ_ACTIVE_INST_VALU "
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_INST_CYCLES_SALU GRBM_GUI_ACTIVE",
    "SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_ANY SQ_WAIT_INST_ANY SQ_BUSY_CYCLES "
    "SQ_ACTIVE_INST_LDS SQ_INSTS_VMEM SQ_ACTIVE_INST_SCA GRBM_GUI_ACTIVE",
]


def counters_by_dispatch(path):
    """{dispatch: (kernel name, {counter: value summed over SEs and XCCs})}."""
    out = {}
    for r in csv.DictReader(open(path)):
        d = int(r["Dispatch_Id"])
        name, vals = out.setdefault(d, (r["Kernel_Name"], {}))
        vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def pmc_summary(pmc1, pmc2, n_xcc=8, cu_active=192, simd_per_cu=4, chunks=4096):
    """Busy fractions and instruction mix of the chunk kernel from two
    counter passes (derived the way rocprofv3's VALUBusy, SALUBusy, MfmaUtil
    and LdsUtil are, over the CUs the kernel occupies)."""
    rows = {}
    for path in (pmc1, pmc2):
        for d, (name, vals) in counters_by_dispatch(path).items():
            if CHUNK_TAG in name:
                rows.setdefault(d, {}).update(vals)
    last = [rows[d] for d in sorted(rows)][-1]
    cycles = last["GRBM_GUI_ACTIVE"] / n_xcc          # per XCC
    per_chunk = lambda c: last[c] / cu_active / chunks
    lines = ["# rocprofv3 counters of the chunk kernel (chunk 16, T=65536, H=96, D=128, bf16), MI355X,",
             "# last of its three dispatches in `python3 bench.py --counters`; two passes:"]
    lines += [f"#   rocprofv3 --pmc {p} -T -f csv -d <dir> -o pmcN -- python3 bench.py --counters"
              for p in PMC_PASSES]
    lines += [f"# {cu_active} CUs active (one workgroup each), {chunks} chunks per workgroup, "
              f"{cycles:.3g} shader cycles per XCC", ""]
    lines.append(f"VALU busy  {100 * last['SQ_ACTIVE_INST_VALU'] / cu_active / cycles:5.1f} % "
                 "(SQ_ACTIVE_INST_VALU over the active CUs)")
    lines.append(f"SALU busy  {100 * last['SQ_INST_CYCLES_SALU'] / cu_active / cycles:5.1f} %")
    lines.append(f"MFMA busy  {100 * last['SQ_VALU_MFMA_BUSY_CYCLES'] / (cu_active * simd_per_cu) / cycles:5.1f} % "
                 "(SQ_VALU_MFMA_BUSY_CYCLES over the active SIMDs)")
    lines.append(f"LDS busy   {100 * last['SQ_LDS_IDX_ACTIVE'] / cu_active / cycles:5.1f} %, of which bank "
                 f"conflicts {100 * last['SQ_LDS_BANK_CONFLICT'] / last['SQ_LDS_IDX_ACTIVE']:4.1f} %")
    lines.append("instructions per chunk per CU: " + ", ".join(
        f"{k[9:].lower()} {per_chunk(k):.0f}" for k in
        ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA", "SQ_INSTS_VMEM")))
    lines.append(f"shader cycles per chunk: {cycles / chunks:.0f}")
    return lines


L2_PASSES = [
    "TCC_HIT_sum TCC_MISS_sum TCC_EA0_WRREQ_STALL_sum TCC_TAG_STALL_sum "
    "TCP_PENDING_STALL_CYCLES_sum TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum "
    "TCP_TCC_WRITE_REQ_sum GRBM_GUI_ACTIVE",
    "TCC_EA0_RDREQ_LEVEL_sum TCC_EA0_RDREQ_sum TCC_EA0_WRREQ_LEVEL_sum TCC_EA0_WRREQ_sum "
    "GRBM_GUI_ACTIVE",
    "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum TCC_BUSY_sum "
    "TCC_CYCLE_sum GRBM_GUI_ACTIVE",
]
# streaming kernels of the counter run compared on their memory path, with the
# tag that finds each one's last dispatch
L2_KERNELS = [
    ("conv bf16 (kda_conv)", "conv_kernelIDF16bLi128ELb0E"),
    ("conv MXFP8 out (kda_conv_mxfp8)", "conv_kernelIDF16bLi128ELb1E"),
    ("gated norm (kda_gated_norm)", "gated_norm_kernel"),
    ("copy, 2 GiB in + 2 GiB out", COPY_TAG),
    ("chunk (kda_chunk_prefill)", CHUNK_TAG),
    ("latent attention over the cache", "mla_attn_kernel"),
]


def memory_path_summary(l2a, l2b, l2c, n_xcc=8, n_cu=256, tcc_instances=128):
    """L1 and L2 request counts, HBM latencies (Little's law: the summed
    request level over the requests) and stall fractions of the streaming
    kernels, from three counter passes of `bench.py --counters`."""
    def last(path, tag):
        d = counters_by_dispatch(path)
        hits = [k for k in sorted(d) if tag in d[k][0]]
        return d[hits[-1]][1] if hits else None

    def times(path, tag):
        t = {}
        for r in csv.DictReader(open(path)):
            if tag in r["Kernel_Name"]:
                t[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6
        return t[max(t)] if t else float("nan")

    lines = ["# Memory path of the streaming kernels: rocprofv3 L1 (TCP) and L2 (TCC) counters, MI355X,",
             "# last dispatch of each kernel in `python3 bench.py --counters`; three passes:"]
    lines += [f"#   rocprofv3 --pmc {p} -T -f csv -d <dir> -o l2{'abc'[i]} -- python3 bench.py --counters"
              for i, p in enumerate(L2_PASSES)]
    lines += ["# cycles: GRBM_GUI_ACTIVE over the 8 XCCs (shader clock); L2 cycles: TCC_CYCLE over its",
              f"# {tcc_instances} instances; latencies in L2 cycles; 'in flight' = requests outstanding at the",
              "# L2-to-memory interface on average (chip-wide), 128-byte reads; L1 requests per cycle are per CU",
              f"# over all {n_cu} CUs; 'L1 pending' = share of CU cycles the L1 waits on outstanding requests", "",
              f"{'kernel':34s} {'ms':>6s} {'L1 rd req':>10s} {'L1 wr req':>10s} {'req/cyc/CU':>10s} "
              f"{'L1 pending':>10s} {'L2 hit':>7s} {'rd lat':>7s} {'wr lat':>7s} {'rd in flight':>12s} "
              f"{'DRAM rd/wr credit stall':>23s}"]
    for label, tag in L2_KERNELS:
        a, b, c = last(l2a, tag), last(l2b, tag), last(l2c, tag)
        if not (a and b and c):
            lines.append(f"{label:34s}  no dispatches")
            continue
        cyc = a["GRBM_GUI_ACTIVE"] / n_xcc
        l2cyc = c["TCC_CYCLE_sum"] / tcc_instances
        rd, wr = a["TCP_TCC_READ_REQ_sum"], a["TCP_TCC_WRITE_REQ_sum"]
        lines.append(
            f"{label:34s} {times(l2a, tag):6.3f} {rd:10.3e} {wr:10.3e} {(rd + wr) / cyc / n_cu:10.3f} "
            f"{100 * a['TCP_PENDING_STALL_CYCLES_sum'] / cyc / n_cu:9.1f}% "
            f"{100 * a['TCC_HIT_sum'] / (a['TCC_HIT_sum'] + a['TCC_MISS_sum']):6.1f}% "
            f"{b['TCC_EA0_RDREQ_LEVEL_sum'] / b['TCC_EA0_RDREQ_sum']:7.0f} "
            f"{b['TCC_EA0_WRREQ_LEVEL_sum'] / b['TCC_EA0_WRREQ_sum']:7.0f} "
            f"{b['TCC_EA0_RDREQ_LEVEL_sum'] / l2cyc:12.0f} "
            f"{100 * c['TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum'] / c['TCC_CYCLE_sum']:10.2f}% / "
            f"{100 * c['TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum'] / c['TCC_CYCLE_sum']:.2f}%")
    return lines


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--pmc1", help="counter_collection.csv of the first counter pass (optional)")
    ap.add_argument("--pmc2", help="counter_collection.csv of the second counter pass")
    ap.add_argument("--l2a", help="counter_collection.csv of the first L1/L2 pass (L2_PASSES)")
    ap.add_argument("--l2b", help="... of the second")
    ap.add_argument("--l2c", help="... of the third")
    args = ap.parse_args()
    if args.l2a and args.l2b and args.l2c:
        ml = memory_path_summary(args.l2a, args.l2b, args.l2c)
        os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
        with open(os.path.join(ROOT, "profiles", "memory_path_T65536.txt"), "w") as f:
            f.write("\n".join(ml) + "\n")
        print("\n".join(ml))
    if not (args.trace and args.fetch and args.write):
        if not args.l2a:
            ap.error("--trace, --fetch and --write are required (or the three --l2 passes)")
        return
    import bench
    if args.pmc1 and args.pmc2:
        pl = pmc_summary(args.pmc1, args.pmc2)
        os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
        with open(os.path.join(ROOT, "profiles", "chunk_prefill_T65536_pmc.txt"), "w") as f:
            f.write("\n".join(pl) + "\n")
        print("\n".join(pl))

    # kernel-trace statistics
    rows = list(csv.DictReader(open(args.trace)))
    lines = ["# rocprofv3 kernel statistics of one bench.py run (prefill T=65536, H=96, D=128,",
             "# bf16 I/O; decode B=256 x 64 steps; latent-attention decode B=256 x 4096), MI355X",
             "# command: rocprofv3 --kernel-trace --stats -T -f csv -d <dir> -o bench -- "
             "python3 bench.py --steps 20 --warmup 10 --no-cpu-baseline",
             f"{'kernel':60s} {'calls':>6s} {'avg_ms':>10s} {'min_ms':>10s} {'max_ms':>10s} {'pct':>6s}"]
    for r in rows:
        lines.append(f"{r['Name'][:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e6:10.4f} "
                     f"{float(r['MinNs'])/1e6:10.4f} {float(r['MaxNs'])/1e6:10.4f} "
                     f"{float(r['Percentage']):6.2f}")
    chunk_avg = [float(r["AverageNs"]) / 1e6 for r in rows if CHUNK_TAG in r["Name"]]
    # per dispatch: bench.py launches the chunk kernel WARMUP + STEPS times
    # for the headline workload (T=65536) first, then as often for each of the
    # other two prefill workloads; the headline's timed steps are launches
    # WARMUP .. WARMUP + STEPS - 1
    WARMUP, STEPS = 10, 20
    ktrace = os.path.join(os.path.dirname(args.trace), "bench_kernel_trace.csv")
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
            for r in csv.DictReader(open(ktrace)) if CHUNK_TAG in r["Kernel_Name"]]
    timed = durs[WARMUP:WARMUP + STEPS]
    timed_avg = statistics.mean(timed) if len(timed) == STEPS else None
    lines += ["", f"# chunk kernel per dispatch (ms): {' '.join(f'{d:.3f}' for d in durs)}",
              f"# chunk kernel average over the {STEPS} timed steps of T=65536 (launches "
              f"{WARMUP + 1}..{WARMUP + STEPS}): " + (f"{timed_avg:.4f} ms" if timed_avg else "n/a")]

    # byte counters
    fetch = per_dispatch(args.fetch, "FETCH_SIZE")
    write = per_dispatch(args.write, "WRITE_SIZE")
    f_chunk = [v for n, v in fetch if CHUNK_TAG in n]
    w_chunk = [v for n, v in write if CHUNK_TAG in n]
    # the copy dispatches are the last three elementwise kernels of the run
    f_copy = [v for n, v in fetch if COPY_TAG in n][-3:]
    w_copy = [v for n, v in write if COPY_TAG in n][-3:]
    f_scale = COPY_BYTES / (statistics.mean(f_copy) * 1024)
    w_scale = COPY_BYTES / (statistics.mean(w_copy) * 1024)
    fb = statistics.mean(f_chunk) * 1024 * f_scale
    wb = statistics.mean(w_chunk) * 1024 * w_scale
    algo = bench.prefill_bytes(65536, 96, 128, 1)["chunk"]
    rec = {
        "kernel": bench.CHUNK_KERNEL + ", T=65536, H=96",
        "source_sha256": bench.chunk_source_hash(),
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE -T -f csv -d <dir> -o fetch -- python3 bench.py --counters",
            "rocprofv3 --pmc WRITE_SIZE -T -f csv -d <dir> -o write -- python3 bench.py --counters",
        ],
        "fetch_kib_per_dispatch": statistics.mean(f_chunk),
        "write_kib_per_dispatch": statistics.mean(w_chunk),
        "copy_calibration": {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                             "fetch_kib": statistics.mean(f_copy),
                             "write_kib": statistics.mean(w_copy),
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "fetch_bytes_per_launch": fb,
        "write_bytes_per_launch": wb,
        "traffic_bytes_per_launch": fb + wb,
        "algorithmic_bytes_per_launch": algo,
        "traffic_over_algorithmic": (fb + wb) / algo,
        "kernel_trace_avg_ms_all_workloads": chunk_avg[0] if chunk_avg else None,
        "kernel_trace_timed_avg_ms": timed_avg,
    }
    lines += ["",
              "# HBM bytes of the chunk kernel from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),",
              "# scaled by the same counters on a copy kernel of 2 GiB in / 2 GiB out:",
              f"#   FETCH_SIZE {rec['fetch_kib_per_dispatch']:.0f} KiB x {f_scale:.3f} = {fb/1e9:.3f} GB",
              f"#   WRITE_SIZE {rec['write_kib_per_dispatch']:.0f} KiB x {w_scale:.3f} = {wb/1e9:.3f} GB",
              f"#   traffic {(fb+wb)/1e9:.3f} GB vs algorithmic {algo/1e9:.3f} GB "
              f"({rec['traffic_over_algorithmic']:.3f}x)"]
    # every kernel of the counter run against its algorithmic bytes
    pb = bench.prefill_bytes(65536, 96, 128, 1)
    kinds = [
        ("conv (kda_conv, T=65536)", "conv_kernelIDF16bLi128ELb0E", pb["conv"]),
        ("chunk (kda_chunk_prefill, chunk 16, T=65536)", CHUNK_TAG, pb["chunk"]),
        ("conv MXFP8 out (kda_conv_mxfp8, T=65536)", "conv_kernelIDF16bLi128ELb1E",
         bench.mxfp8_conv_bytes(65536, 96, 128)),
        ("chunk MXFP8 (kda_chunk_prefill_mxfp8, T=65536)", MX_TAG,
         bench.mxfp8_chunk_bytes(65536, 96, 128, 1)),
        ("fused conv+chunk (kda_prefill_fused, T=65536)", CV_TAG, pb["chunk"]),
        ("gated norm (kda_gated_norm, T=65536)", "gated_norm_kernel", pb["norm"]),
        ("decode, 1 token (kda_decode_step, B=256)", "decode_multi_kernelIDF16bLi128ELb1",
         bench.decode_bytes(256, 96, 128)),
        ("decode, 4 tokens (kda_decode_multi, B=256)", "decode_multi_kernelIDF16bLi128ELb0",
         bench.decode_multi_bytes(256, 4, 96, 128)),
    ]
    # the latent-attention decode step (256 sequences x 4096 cached latents,
    # 96 heads, one split per sequence): each kernel against the bytes it must
    # move, the hand-over between attention and combine included (with one
    # split that is u = U / l in bf16; the (m, l) pair the attention kernel
    # also writes, 0.2 MB, is counted as its own overhead)
    B, H, L, R, Dh = 256, 96, 4096, 512, 128
    partials = B * H * R * 2
    kinds += [
        ("latent attn: absorb (q' = W_uk^T q)", "mla_absorb_kernel",
         B * H * Dh * 2 + H * Dh * R * 2 + B * H * R * 2),
        ("latent attn: attention over the cache", "mla_attn_kernel",
         B * L * R * 2 + B * H * R * 2 + partials),
        ("latent attn: combine (o = W_uv u, gate)", "mla_combine_kernel",
         partials + H * Dh * R * 2 + 2 * B * H * Dh * 2),
    ]
    table = ["# HBM bytes per dispatch from rocprofv3 FETCH_SIZE and WRITE_SIZE (two runs of",
             "#   python3 bench.py --counters), scaled by the same counters on a copy kernel",
             f"#   of 2 GiB in / 2 GiB out (fetch x{f_scale:.3f}, write x{w_scale:.3f}), MI355X",
             "# commands: rocprofv3 --pmc FETCH_SIZE -T -f csv -d <dir> -o fetch -- python3 bench.py --counters",
             "#           rocprofv3 --pmc WRITE_SIZE -T -f csv -d <dir> -o write -- python3 bench.py --counters",
             f"{'kernel':46s} {'n':>2s} {'fetch_GB':>9s} {'write_GB':>9s} {'traffic_GB':>10s} "
             f"{'algo_GB':>9s} {'ratio':>6s}"]
    for label, tag, algo_b in kinds:
        fk = [v for n, v in fetch if tag in n]
        wk = [v for n, v in write if tag in n]
        if not fk or not wk:
            table.append(f"{label:46s}  no dispatches")
            continue
        fbk = statistics.mean(fk) * 1024 * f_scale
        wbk = statistics.mean(wk) * 1024 * w_scale
        table.append(f"{label:46s} {len(fk):2d} {fbk/1e9:9.3f} {wbk/1e9:9.3f} {(fbk+wbk)/1e9:10.3f} "
                     f"{algo_b/1e9:9.3f} {(fbk+wbk)/algo_b:6.3f}")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "kernels_traffic_T65536_B256.txt"), "w") as f:
        f.write("\n".join(table) + "\n")
    print("\n".join(table))
    with open(os.path.join(ROOT, "profiles", "chunk_prefill_T65536_kernel_stats.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(bench.TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=2)
    print("\n".join(lines))


if __name__ == "__main__":
    main()
