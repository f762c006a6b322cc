"""The compiled MFMA kernels never read one MFMA's result as the accumulator
(srcC) of an MFMA of another shape within a few wait states.

On gfx950 a v_mfma_f32_16x16x16_bf16 result read as the accumulator of a
v_mfma_f32_16x16x32_bf16 with no wait states between them comes out wrong,
and the compiler inserts none there (it treats a fully overlapping
accumulator as forwarded, which holds between products of one shape).  The
chunk kernel once fed V into its R chain that way and was right or wrong
depending on the schedule.  This test compiles the MFMA kernels for gfx950
(no GPU needed) and checks the straight-line distance of every such read;
the scanner itself is checked on planted listings.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from linear_attention_recurrence_09_amd import build as kbuild

MIN_WAIT_STATES = 16
KERNELS = ["kda_chunk_pipe.hip", "kda_chunk.hip", "kda_mla.hip"]


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def mixed_srcc_reads(asm_text):
    """(function, writer opcode, reader opcode, wait states) for every MFMA
    whose accumulator operand overlaps the result of an earlier MFMA of a
    different opcode, counted along the listing (s_nop n counts n + 1, any
    other instruction 1; a later MFMA that overwrites the registers ends the
    writer's reach)."""
    found = []
    fn = None
    live = []   # [opcode, result registers, wait states since]
    for raw in asm_text.splitlines():
        line = raw.strip()
        if not line or line.startswith(";"):
            continue
        if re.match(r"^[A-Za-z_][\w.$]*:", line) and not line.startswith(".L"):
            fn, live = line.split(":")[0], []
            continue
        if line.startswith(".") or line.endswith(":"):
            continue
        op = line.split()[0]
        inc = int(line.split()[1]) + 1 if op == "s_nop" else 1
        if op.startswith("v_mfma"):
            ops = [o.strip() for o in line.split(None, 1)[1].split(",")]
            src_c = _regs(ops[3]) if len(ops) > 3 else set()
            for w_op, w_regs, ws in live:
                if w_op != op and src_c & w_regs:
                    found.append((fn, w_op, op, ws))
            dst = _regs(ops[0])
            live = [[o, r, w] for o, r, w in live if not (r & dst)]
            live = [[o, r, w + 1] for o, r, w in live]
            live.append([op, dst, 0])
        else:
            live = [[o, r, w + inc] for o, r, w in live]
        live = [e for e in live if e[2] < 64]
    return found


def test_scanner_flags_a_planted_read():
    asm = """
kernel_a:
\tv_mfma_f32_16x16x16_bf16 v[10:13], v[0:1], v[2:3], 0
\tv_mfma_f32_16x16x32_bf16 v[10:13], v[4:7], v[20:23], v[10:13]
kernel_b:
\tv_mfma_f32_16x16x32_bf16 v[30:33], v[4:7], v[20:23], 0
\ts_nop 7
\ts_nop 7
\tv_add_f32_e32 v1, v2, v3
\tv_mfma_f32_16x16x16_bf16 v[30:33], v[0:1], v[2:3], v[30:33]
kernel_c:
\tv_mfma_f32_16x16x32_bf16 v[40:43], v[4:7], v[20:23], 0
\tv_mfma_f32_16x16x32_bf16 v[40:43], v[8:11], v[24:27], v[40:43]
"""
    found = mixed_srcc_reads(asm)
    assert ("kernel_a", "v_mfma_f32_16x16x16_bf16", "v_mfma_f32_16x16x32_bf16", 0) in found
    assert ("kernel_b", "v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x16_bf16", 17) in found
    assert not [f for f in found if f[0] == "kernel_c"]   # one shape: forwarded


def _compile_to_asm(src, out_dir):
    out = os.path.join(out_dir, os.path.splitext(src)[0] + ".s")
    cmd = [kbuild.HIPCC, *kbuild.COMMON, "-x", "hip", "-S", "--cuda-device-only",
           os.path.join(kbuild.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.mark.skipif(not shutil.which(kbuild.HIPCC) and not os.path.exists(kbuild.HIPCC),
                    reason="hipcc not available")
def test_no_mixed_shape_accumulator_read_within_a_few_wait_states(tmp_path):
    with cf.ThreadPoolExecutor(max_workers=len(KERNELS)) as ex:
        texts = dict(zip(KERNELS, ex.map(lambda k: _compile_to_asm(k, str(tmp_path)), KERNELS)))
    bad = []
    n_checked = 0
    for src, text in texts.items():
        for fn, w_op, r_op, ws in mixed_srcc_reads(text):
            n_checked += 1
            if ws < MIN_WAIT_STATES:
                bad.append(f"{src} {fn[:90]}: {w_op} -> accumulator of {r_op} after {ws}")
    # the chunk kernel's A_qk product onto the O^T chain is such a read in
    # every instantiation, so the scan must find some
    assert n_checked > 0
    assert not bad, "\n".join(bad)
