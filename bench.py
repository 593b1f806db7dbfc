"""Benchmark of the Comba hot path on one MI355X.

One step = one comba_chunk_fwd over the 1.3B-layer batch (B=8, H=16,
T=4096, K=V=128, bf16 q/k/v/o, fp32 alpha/beta/state, non-zero initial
state), inputs resident in device memory (two copies used in turn, so that the
last-level cache cannot serve one step from the last). The reported value is sequence
tokens (B*T) per second, the mean over the timed steps; the median of runs of
ten steps is reported beside it. The part's own ceilings (an elementwise kernel's
HBM rate, a bf16 matrix-core loop) are measured first, which also brings the
clocks up, and the headline leg always warms up for at least
HEADLINE_WARMUP_FLOOR launches, whatever --warmup asks for.

Also timed, as context: the 340M layer (B=4, T=2048, H=16) and the packed
batch of 64 lognormal-length sequences (H=32, K=V=64) under "configs"; the
decode step (256 sequences x 16 heads, K=V=128, fp32 state updated in place
in device memory) in GB/s under "decode"; the 1.3B layer with input-side
fusion (raw q/k normalised in the kernel, alpha/beta given as logits) under
"fused", beside the same preprocessing done by separate torch ops before an
unfused call; the 64K-token single-sequence workload plain and
segment-parallel under "long_context"; the 1.3B layer with one q/k head
shared by all value heads under "shared_qk"; and the layer's chunk backward
under "backward". The fp64 CPU oracle is timed on the host cores on a bounded
sample of the headline workload ("cpu_baseline"); its first pass over the
whole batch also checks the benchmarked output ("parity").

Prints one JSON line. Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]

Counter calibration: run under `rocprofv3 --pmc FETCH_SIZE` and again under
`--pmc WRITE_SIZE` with --calibrate-copy (a plain 256 MiB device-to-device
copy follows the timed work), then `python bench.py --record-traffic
<fetch_dir> <write_dir>` turns the two counter tables into the HBM bytes per
launch of the chunk kernel and of the decode kernel, scaled by what the same
counter reads for the copy.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 matrix-core peak (256 CU x 2.4 GHz x 4096 flop/clk)
CHUNK = 64


def chunk_fwd_algorithmic(B, T, H, K, V, with_s0=True, num_seqs=None):
    """Bytes and flops that any implementation must move / perform.

    Bytes: q, k (K bf16), v, o (V bf16), alpha, beta (fp32) per head-token,
    plus the initial (if any) and final fp32 state once per (sequence, head);
    B * T is the total token count (B = 1 for a packed batch of num_seqs).
    Flops (triangle-aware chunk form, per chunk of C tokens): C(C-1)K for
    K K^T, C(C+1)K for Q K^T, C(C+1)K for W, C(C+1)V for U, 6CKV for
    W h, the state update and Q h, C(C+1)V for the intra-chunk output and
    C^3/3 for the inverse.
    """
    ht = B * T * H
    nseq = B if num_seqs is None else num_seqs
    nbytes = ht * (2 * K * 2 + 2 * V * 2 + 8) + (2 if with_s0 else 1) * nseq * H * V * K * 4
    C = CHUNK
    per_chunk = (C * (C - 1) * K + C * (C + 1) * K + C * (C + 1) * K + C * (C + 1) * V
                 + 6 * C * K * V + C * (C + 1) * V + C ** 3 / 3)
    flops = per_chunk / C * ht
    return nbytes, flops


def chunk_bwd_algorithmic(B, T, H, K, V):
    """Bytes and flops of the chunk backward at the algorithm's floor.

    Bytes: q, k, v, dO (bf16), alpha, beta (fp32) read once and dq, dk, dv,
    dalpha, dbeta (fp32) written once per head-token, plus S0 and dS_final
    read and dS0 written once per (sequence, head). Checkpoints, the cached
    inverse and score matrices and every re-read are design traffic beyond it.
    Flops (per chunk of C tokens, triangle-aware as for the forward): forming
    Ubar from the chunk's state (K h, Tinv R), dUbar = P^T dO + e^(Gn-G) K dh,
    dR = Tinv^T dUbar, dh_in = q~^T diag(e^G) dO - K^T diag(b1) dR, dA, dP,
    dO h^T, dR h^T, Ubar dh^T, (dP (.) M) K, (dP (.) M)^T q~, beta W K and
    W^T beta K; the chunk inverse (cached or recomputed) is not counted.
    """
    ht = B * T * H
    nbytes = ht * (2 * K * 2 + 2 * V * 2 + 8) + ht * (2 * K * 4 + V * 4 + 8) + 3 * B * H * V * K * 4
    C = CHUNK
    per_chunk = (14 * C * K * V + 4 * C * (C + 1) * V + C * (C - 1) * V
                 + 2 * C * (C + 1) * K + 2 * C * (C - 1) * K)
    flops = per_chunk / C * ht
    return nbytes, flops


# the sources the counted chunk-forward kernel is compiled from
FWD_SOURCES = ("chunk_fwd_bf16.hip", "bf16_tiles.h", "chunk_common.h", "device_common.h", "launch.h")


# the sources the counted decode kernel is compiled from
DECODE_SOURCES = ("recurrent_step.hip", "device_common.h", "launch.h")


def kernel_source_hash(files=FWD_SOURCES):
    csrc = os.path.join(ROOT, "bilinear_rnn_amd", "csrc")
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(src_hash, path=None):
    """HBM bytes per launch of a counted kernel (the chunk kernel unless
    another summary is named) from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source."""
    try:
        rec = json.load(open(path or COUNTERS_JSON))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


COPY_CAL_BYTES = 256 << 20
COUNTERS_JSON = os.path.join(ROOT, "profiles", "chunk_fwd_bf16_layer_1p3b_counters.json")
DECODE_COUNTERS_JSON = os.path.join(ROOT, "profiles", "recurrent_decode_counters.json")


def calibration_copy(torch, dev):
    """An elementwise device copy of COPY_CAL_BYTES read and COPY_CAL_BYTES
    written (fp32 -> int32, so that it runs as a kernel rather than a DMA
    transfer), three times: the known-size reference the HBM byte counters
    are scaled by."""
    src = torch.empty(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty(COPY_CAL_BYTES // 4, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def _counter_rows(d):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def _is_plain_chunk(name):
    # the plain instantiation: no in-kernel normalisation, not state-only
    return "chunk_fwd_bf16_kernel<" in name and "unsigned short, false, false>" in name


def _is_decode(name):
    return "recurrent_kernel<" in name


def _kernel_and_copy(rows, counter, is_kernel=_is_plain_chunk):
    """Mean counter value (KiB per dispatch) of the counted kernel, and of the
    calibration copy: the one kernel dispatched exactly three times after the
    last dispatch of any counted kernel (chunk or decode)."""
    import collections
    rows = [r for r in rows if r["Counter_Name"] == counter]
    is_ker = lambda r: is_kernel(r["Kernel_Name"])
    ker = [float(r["Counter_Value"]) for r in rows if is_ker(r)]
    if not ker:
        return None
    last = max(int(r["Dispatch_Id"]) for r in rows if _is_plain_chunk(r["Kernel_Name"]) or _is_decode(r["Kernel_Name"]))
    groups = collections.defaultdict(list)
    for r in rows:
        if int(r["Dispatch_Id"]) > last:
            groups[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    cal = [(name, v) for name, v in groups.items() if len(v) == 3]
    if len(cal) != 1:
        raise SystemExit(f"cannot identify the calibration copy among {[(n[:60], len(v)) for n, v in groups.items()]}")
    name, v = cal[0]
    return sum(ker) / len(ker), len(ker), sum(v) / len(v), len(v), name


def record_traffic(fetch_dir, write_dir):
    """Write the calibrated per-launch HBM traffic of the chunk kernel and, if
    the counted run had decode steps, of the decode kernel."""
    frows, wrows = _counter_rows(fetch_dir), _counter_rows(write_dir)
    _record_one(frows, wrows, _is_plain_chunk, COUNTERS_JSON,
                "chunk_fwd_bf16_kernel<128,128,64> on layer_1p3b (B=8 T=4096 H=16 K=V=128)",
                kernel_source_hash(), chunk_fwd_algorithmic(8, 4096, 16, 128, 128)[0])
    from bilinear_rnn_amd.inputs import WORKLOADS
    wd = WORKLOADS["decode"]
    ht = wd.B * wd.H
    _record_one(frows, wrows, _is_decode, DECODE_COUNTERS_JSON,
                f"recurrent_kernel<{wd.K},{wd.V},32,bf16,bf16> on the decode workload ({wd.B} x {wd.H} heads, K={wd.K} V={wd.V})",
                kernel_source_hash(DECODE_SOURCES), 2 * ht * wd.V * wd.K * 4 + ht * (2 * wd.K * 2 + 2 * wd.V * 2 + 8))
    record_bwd_traffic(frows, wrows)


BWD_COUNTERS_JSON = os.path.join(ROOT, "profiles", "chunk_bwd_layer_1p3b_counters.json")
BWD_SOURCES = ("chunk_bwd.hip", "chunk_fwd_bf16.hip", "chunk_common.h", "device_common.h", "bf16_tiles.h",
               "launch.h")
BWD_KERNELS = (("checkpointing forward", "chunk_fwd_bf16_kernel<128, 128, 64, unsigned short, false, true>"),
               ("prep", "chunk_bwd_prep_kernel<128, unsigned short>"),
               ("reverse scan", "chunk_bwd_dh_pc_kernel<128, 128>"),
               ("gradient pass", "chunk_bwd_grad_bf16_kernel<128, 128>"),
               ("dd reduction", "dd_reduce_kernel"))


def record_bwd_traffic(frows, wrows):
    """Calibrated HBM bytes per launch of each kernel of the 1.3B-layer
    backward, and their sum against the backward's algorithmic floor."""
    out = {"kernels": {}, "kernel_source_hash": kernel_source_hash(BWD_SOURCES)}
    total = 0.0
    for label, pat in BWD_KERNELS:
        f = _kernel_and_copy(frows, "FETCH_SIZE", lambda n, p=pat: p in n)
        w = _kernel_and_copy(wrows, "WRITE_SIZE", lambda n, p=pat: p in n)
        if f is None or w is None:
            continue
        rd = f[0] * 1024.0 * COPY_CAL_BYTES / (f[2] * 1024.0)
        wr = w[0] * 1024.0 * COPY_CAL_BYTES / (w[2] * 1024.0)
        out["kernels"][label] = {"kernel": pat, "hbm_read_bytes": rd, "hbm_write_bytes": wr, "dispatches": [f[1], w[1]]}
        total += rd + wr
    if not out["kernels"]:
        print("no backward dispatches in the counted runs")
        return
    out["hbm_bytes_per_backward"] = total
    out["algorithmic_bytes"] = chunk_bwd_algorithmic(8, 4096, 16, 128, 128)[0]
    out["traffic_over_algorithmic"] = total / out["algorithmic_bytes"]
    with open(BWD_COUNTERS_JSON, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out, indent=1))


def _record_one(frows, wrows, is_kernel, path, label, src_hash, nbytes):
    got_f, got_w = _kernel_and_copy(frows, "FETCH_SIZE", is_kernel), _kernel_and_copy(wrows, "WRITE_SIZE", is_kernel)
    if got_f is None or got_w is None:
        print(f"no dispatches of {label.split()[0]} in the counted runs: {os.path.basename(path)} not written")
        return
    kf, nkf, cf, ncf, cname = got_f
    kw, nkw, cw, ncw, _ = got_w
    f_scale = COPY_CAL_BYTES / (cf * 1024.0)   # counter KiB -> true bytes, from the copy's read side
    w_scale = COPY_CAL_BYTES / (cw * 1024.0)
    rec = {
        "kernel": label,
        "kernel_source_hash": src_hash,
        "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw,
        "kernel_dispatches": [nkf, nkw],
        "copy_kernel": cname, "copy_bytes": COPY_CAL_BYTES,
        "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_dispatches": [ncf, ncw],
        "fetch_scale": f_scale, "write_scale": w_scale,
        "hbm_read_bytes_per_launch": kf * 1024.0 * f_scale,
        "hbm_write_bytes_per_launch": kw * 1024.0 * w_scale,
    }
    rec["hbm_bytes_per_launch"] = rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
    rec["algorithmic_bytes_per_launch"] = nbytes
    rec["traffic_over_algorithmic"] = rec["hbm_bytes_per_launch"] / nbytes
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


# Per-wave SQ counters: collected in passes of at most eight SQ counters each
# (one --pmc run per pass), then summarised by --summarize-counters.
SQ_PASSES = (
    "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_SMEM SQ_INSTS_VMEM SQ_INSTS_BRANCH "
    "GRBM_GUI_ACTIVE",
    "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY "
    "SQ_WAIT_INST_ANY SQ_WAIT_ANY GRBM_GUI_ACTIVE",
    "SQ_WAVES SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_SCA "
    "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE",
)


def summarize_counters(dirs, kernel_regex, out_md, title, command):
    """Mean value per dispatch of every counter in the rocprofv3 --pmc runs
    under ``dirs``, for the kernels whose names match ``kernel_regex``, and the
    per-wave figures derived from them; written as a markdown table."""
    import re
    import collections
    rx = re.compile(kernel_regex)
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in dirs:
        for r in _counter_rows(d):
            if rx.search(r["Kernel_Name"]):
                vals[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = [f"# {title}", "", "Commands (repository root on the GPU host; one --pmc pass per line):", "", "```"]
    lines += [command.format(i=i, counters=c) for i, c in enumerate(SQ_PASSES)]
    lines += ["```", ""]
    for name, cs in sorted(vals.items()):
        m = {c: sum(v) / len(v) for c, v in cs.items()}
        n = {c: len(v) for c, v in cs.items()}
        short = re.split(r"\((?!anonymous namespace\))", name, maxsplit=1)[0]
        lines += [f"## `{short}`", "", "| Counter | Mean per dispatch | Dispatches |", "|---|---|---|"]
        lines += [f"| {c} | {m[c]:,.0f} | {n[c]} |" for c in sorted(m)]
        w = m.get("SQ_WAVES")
        if w:
            lines += ["", "Per wavefront (counter / SQ_WAVES):", ""]
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_SMEM",
                      "SQ_INSTS_VMEM", "SQ_INSTS_BRANCH"):
                if c in m:
                    lines.append(f"- {c}: {m[c] / w:,.0f}")
            if "SQ_INSTS_VALU" in m and "SQ_INSTS_MFMA" in m:
                lines.append(f"- VALU other than MFMA: {(m['SQ_INSTS_VALU'] - m['SQ_INSTS_MFMA']) / w:,.0f}")
        g = m.get("GRBM_GUI_ACTIVE")
        if g:
            cyc = g / 8.0  # GRBM_GUI_ACTIVE is summed over the 8 XCDs
            lines += ["", f"Derived (kernel length = GRBM_GUI_ACTIVE / 8 XCDs = {cyc:,.0f} cycles; 1024 SIMDs):", ""]
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                lines.append(f"- matrix cores busy: {m['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 1024):.1%} of SIMD cycles "
                             "(SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024))")
            if "SQ_ACTIVE_INST_VALU" in m:
                lines.append(f"- VALU issue (MFMA issue included) busy: "
                             f"{4 * m['SQ_ACTIVE_INST_VALU'] / (cyc * 1024):.1%} of SIMD cycles "
                             "(4 x SQ_ACTIVE_INST_VALU quad-cycles / (cycles x 1024))")
            if m.get("SQ_WAVE_CYCLES"):
                for c, what in (("SQ_ACTIVE_INST_ANY", "issuing an instruction"),
                                ("SQ_WAIT_INST_ANY", "waiting for an instruction's operands (s_waitcnt)"),
                                ("SQ_WAIT_ANY", "waiting for anything else (barriers, sleeps)")):
                    if c in m:
                        lines.append(f"- wavefronts {what}: {m[c] / m['SQ_WAVE_CYCLES']:.1%} of wave cycles "
                                     f"({c} / SQ_WAVE_CYCLES)")
            if m.get("SQ_LDS_IDX_ACTIVE"):
                lines.append(f"- LDS bank-conflict cycles: {m['SQ_LDS_BANK_CONFLICT'] / m['SQ_LDS_IDX_ACTIVE']:.1%} "
                             "of LDS-active cycles (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE)")
        lines.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def device_inputs(inp, torch, dev):
    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def f32(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)

    cu = None
    if inp.cu_seqlens is not None:
        cu = torch.from_numpy(np.ascontiguousarray(inp.cu_seqlens, dtype=np.int32)).to(dev)
    return dict(q=bf16(inp.q_bits), k=bf16(inp.k_bits), v=bf16(inp.v_bits), alpha=f32(inp.alpha),
                beta=f32(inp.beta), d=f32(inp.d), s0=f32(inp.s0), cu=cu)


# Every timed leg first runs its step for at least this long (and at least
# --warmup launches): the first tens of milliseconds of launches after idle or
# after other work run up to 15 % slower while the clock settles.
WARMUP_FLOOR_S = 0.06


def time_loop(torch, fn, steps, warmup, floor_s=None):
    """Mean time of one call of fn (ms) over `steps` back-to-back calls timed
    with events on the launch stream, after at least `warmup` untimed calls
    and at least `floor_s` seconds of them; and the wall time of the timed
    calls."""
    floor_s = WARMUP_FLOOR_S if floor_s is None else floor_s
    t_w = time.perf_counter()
    nwarm = 0
    while nwarm < warmup or time.perf_counter() - t_w < floor_s:
        fn(nwarm)
        nwarm += 1
        if nwarm % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    time_loop.last_warmup = nwarm
    return start.elapsed_time(end) / steps, wall


def step_distribution(torch, fn, groups=30, per_group=10):
    """Spread of the step time: `groups` runs of `per_group` back-to-back
    steps, each run bracketed by its own events on the launch stream; the
    median, p10 and p90 of the per-step time of a run (us). Reported beside
    the timed mean, not used for it; runs of several steps keep the events'
    own cost out of the figure."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(groups)]
    torch.cuda.synchronize()
    for g, (a, b) in enumerate(ev):
        a.record(stream)
        for i in range(per_group):
            fn(g * per_group + i)
        b.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 / per_group for a, b in ev])
    return {"median": float(np.median(us)), "p10": float(np.percentile(us, 10)),
            "p90": float(np.percentile(us, 90)), "runs": groups, "steps_per_run": per_group}


# The headline leg always warms up for at least this many launches and this
# long (about 0.1 s), whatever --warmup asks for: measured on the part, launches
# 100-200 after a cold start still run about 2 % slower than 200-300.
HEADLINE_WARMUP_FLOOR = 200
HEADLINE_WARMUP_S = 0.1

PEAK_COPY_BYTES = 512 << 20     # twice the 256 MB last-level cache
PEAK_PROBE_BLOCKS = 2048        # eight workgroups of four wavefronts per compute unit
PEAK_PROBE_ITERS = 4096


def measured_peaks(torch, comba, dev):
    """The part's own ceilings, measured in the same run: HBM bandwidth of an
    out-of-place and of an in-place elementwise scale over 512 MiB fp32
    buffers, and the bf16 matrix-core rate of the library's MFMA loop."""
    n = PEAK_COPY_BYTES // 4
    src = torch.empty(n, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    cms, _ = time_loop(torch, lambda i: torch.mul(src, 1.0, out=dst), 20, 5)
    ims, _ = time_loop(torch, lambda i: src.mul_(1.0), 20, 5)
    del src, dst
    sink = torch.empty(PEAK_PROBE_BLOCKS * 256, dtype=torch.float32, device=dev)
    flops = PEAK_PROBE_BLOCKS * PEAK_PROBE_ITERS * comba.api.PEAK_PROBE_FLOPS_PER_BLOCK_ITER
    pms, _ = time_loop(torch, lambda i: comba.mfma_peak_probe(sink, PEAK_PROBE_ITERS), 10, 3)
    del sink
    return {"hbm_copy_GB/s": 2 * PEAK_COPY_BYTES / (cms * 1e-3) / 1e9,
            "hbm_inplace_GB/s": 2 * PEAK_COPY_BYTES / (ims * 1e-3) / 1e9,
            "mfma_bf16_TFLOP/s": flops / (pms * 1e-3) / 1e12,
            "how": f"out-of-place and in-place fp32 scale of {PEAK_COPY_BYTES >> 20} MiB (bytes read + written); "
                   f"comba_mfma_peak_probe, {PEAK_PROBE_BLOCKS} workgroups x {PEAK_PROBE_ITERS} iterations"}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, H, gpu_out=None, min_seconds=10.0):
    """fp64 C oracle on all host cores, whole-batch passes repeated until at
    least ``min_seconds`` of wall time (bounded: one pass is about half a
    second on 16 cores). Reported in sequence tokens per second.

    ``gpu_out`` = (o, final_state) of the benchmarked launch, host float arrays:
    the first pass's output then also checks it over the whole batch (rel-L2 and
    the worst token-head row of o; the same for the final state). Returns
    (baseline, parity or None)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    nthreads = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
    B, T = inp.q.shape[0], inp.q.shape[1]
    args = [np.ascontiguousarray(x, dtype=np.float64) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.d)]
    s0 = np.ascontiguousarray(inp.s0, dtype=np.float64)
    passes = 0
    parity = None
    t0 = time.perf_counter()
    while True:
        ro, rs = oracle.comba_forward_c(*args, s0, None, nthreads=nthreads)
        passes += 1
        if passes == 1 and gpu_out is not None:
            t_chk = time.perf_counter()
            o, sf = gpu_out
            parity = {"o_rel_l2": oracle.rel_l2(o, ro), "o_worst_row": oracle.row_rel_err(o, ro),
                      "state_rel_l2": oracle.rel_l2(sf, rs), "state_worst_row": oracle.row_rel_err(sf, rs),
                      "gates": {"o_rel_l2": 2e-3, "o_worst_row": 2.0 ** -8 + 1e-3, "state_rel_l2": 2e-3,
                                "state_worst_row": 1e-3},
                      "checked": f"whole batch: all {B} x {H} (sequence, head) pairs, every token"}
            parity["ok"] = (parity["o_rel_l2"] <= 2e-3 and parity["o_worst_row"] <= 2.0 ** -8 + 1e-3
                            and parity["state_rel_l2"] <= 2e-3 and parity["state_worst_row"] <= 1e-3)
            t0 += time.perf_counter() - t_chk  # the comparison is not oracle time
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    # one core, on one batch row (all heads), repeated for at least 2 s
    one = [a[:1] for a in args[:5]] + [args[5]]
    p1 = 0
    t1 = time.perf_counter()
    while True:
        oracle.comba_forward_c(*one, s0[:1], None, nthreads=1)
        p1 += 1
        d1 = time.perf_counter() - t1
        if d1 >= 2.0:
            break
    base = {"value": passes * B * T / dt, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{passes} passes over the whole batch B={B} T={T} H={H} K=V={inp.q.shape[3]}, "
                      f"fp64 C oracle, {dt:.1f} s wall",
            "cpu_model": _cpu_model(),
            "single_core_tokens/s": p1 * T / d1,
            "single_core_sample": f"{p1} passes over one batch row (T={T}, H={H}), {d1:.1f} s wall"}
    return base, parity


def config_leg(torch, comba, dev, name, steps, warmup, copies):
    """A further forward workload timed like the headline: `copies` resident
    copies of the inputs and outputs used in turn (together larger than the
    256 MB last-level cache), tokens/s and the fractions of the HBM and
    matrix-core rooflines."""
    from bilinear_rnn_amd.inputs import WORKLOADS, make_inputs
    w = WORKLOADS[name]
    inp = make_inputs(w)
    B, T = inp.q.shape[0], inp.q.shape[1]
    H, K, V, N = w.H, w.K, w.V, inp.num_seqs
    tin = [device_inputs(inp, torch, dev) for _ in range(copies)]
    tout = [(torch.empty((B, T, H, V), dtype=torch.bfloat16, device=dev),
             torch.empty((N, H, V, K), dtype=torch.float32, device=dev)) for _ in range(copies)]
    packed = inp.cu_seqlens is not None
    nws = comba.workspace_size(B, T, H, K, V, N if packed else 0)
    ws = torch.empty((max(nws, 1),), dtype=torch.uint8, device=dev)

    def st(i):
        c, (oo, ss) = tin[i % copies], tout[i % copies]
        comba.chunk_fwd(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["d"], c["s0"], c["cu"], out=oo,
                        final_state=ss, workspace=ws)

    ms, _ = time_loop(torch, st, steps, warmup)
    nbytes, flops = chunk_fwd_algorithmic(B, T, H, K, V, with_s0=inp.s0 is not None,
                                          num_seqs=N if packed else None)
    secs = ms * 1e-3
    out = {"workload": name, "B": B, "T": T, "H": H, "K": K, "V": V, "num_seqs": N,
           "tokens": B * T, "us_per_step": ms * 1e3, "tokens/s": B * T / secs,
           "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
           "hbm_frac": nbytes / secs / 1e9 / HBM_PEAK_GBS,
           "mfma_frac": flops / secs / 1e12 / BF16_PEAK_TFLOPS,
           "copies": copies, "step_us": step_distribution(torch, st)}
    if packed:
        lens = np.diff(inp.cu_seqlens)
        out["lengths"] = {"min": int(lens.min()), "median": float(np.median(lens)), "max": int(lens.max()),
                          "seed": w.seed}
    del tin, tout, ws
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-configs", action="store_true", help="skip the 340M-layer and packed-batch legs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured copy / MFMA ceilings")
    ap.add_argument("--no-fused", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-shared-qk", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="finish with a plain 256 MiB device copy (counter calibration runs)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: summarise two rocprofv3 --pmc runs into the counters file")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                    help="no GPU work: per-dispatch means of the SQ counter passes under the given directories")
    ap.add_argument("--kernel-regex", default="comba::")
    ap.add_argument("--out", help="markdown file written by --summarize-counters")
    ap.add_argument("--title", default="SQ counters")
    ap.add_argument("--command", default="", help="the counted command, with {i} and {counters} placeholders")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.kernel_regex, args.out or os.devnull, args.title,
                           args.command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a built feature.", file=sys.stderr)
        sys.exit(2)

    import torch
    import bilinear_rnn_amd as comba
    from bilinear_rnn_amd.inputs import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    w = WORKLOADS["layer_1p3b"]
    inp = make_inputs(w)
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V

    # The part's own ceilings first: they also bring the clocks up before any
    # timed leg (the first tens of milliseconds of launches after idle run up
    # to 15 % slower).
    peaks = None if args.no_peaks else measured_peaks(torch, comba, dev)

    # Two resident copies of the inputs and outputs (2 x 0.56 GB), used in turn, so
    # that the 256 MB last-level cache cannot carry one step's operands into the next.
    fwd_copies = [device_inputs(inp, torch, dev) for _ in range(2)]
    fwd_outs = [(torch.empty((B, T, H, V), dtype=torch.bfloat16, device=dev),
                 torch.empty((B, H, V, K), dtype=torch.float32, device=dev)) for _ in range(2)]
    t = fwd_copies[0]
    o, sf = fwd_outs[0]

    def step(i):
        c, (oo, ss) = fwd_copies[i % 2], fwd_outs[i % 2]
        comba.chunk_fwd(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["d"], c["s0"], out=oo, final_state=ss)

    warm = max(args.warmup, HEADLINE_WARMUP_FLOOR)
    ms, wall = time_loop(torch, step, args.steps, warm, floor_s=HEADLINE_WARMUP_S)
    warm_done = time_loop.last_warmup
    nbytes, flops = chunk_fwd_algorithmic(B, T, H, K, V)
    secs = ms * 1e-3
    achieved = nbytes / secs / 1e9
    src_hash = kernel_source_hash()
    traffic = measured_traffic(src_hash)
    spread = step_distribution(torch, step)

    result = {
        "metric": "Comba chunk-fwd tokens/sec @H16 d128 T4096 + % MFMA roofline; decode GB/s",
        "value": B * T / secs,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_launches": warm_done,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), alpha=sigmoid(N(3,0.5)), "
                "beta=sigmoid(N(0,1)), d=0.5, S0~N(0,0.02))",
        "config": {"workload": "layer_1p3b", "B": B, "T": T, "H": H, "K": K, "V": V, "chunk": CHUNK,
                   "in_dtype": "bf16", "out_dtype": "bf16", "state_dtype": "fp32"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "chunk_fwd_bf16_kernel<128,128,64>", "algorithmic_bytes": nbytes},
        "mfma": {"algorithmic_tflops": flops / secs / 1e12, "peak_tflops": BF16_PEAK_TFLOPS,
                 "frac": flops / secs / 1e12 / BF16_PEAK_TFLOPS, "algorithmic_flops": flops},
        "kernel_source_hash": src_hash,
        "wall_s_timed": wall,
        "step_us": spread,
        "value_at_median_step": B * T / (spread["median"] * 1e-6),
    }
    if peaks is not None:
        result["measured_peaks"] = peaks
        result["roofline"]["frac_of_measured_hbm"] = achieved / max(peaks["hbm_copy_GB/s"], peaks["hbm_inplace_GB/s"])
        result["mfma"]["frac_of_measured"] = flops / secs / 1e12 / peaks["mfma_bf16_TFLOP/s"]
    # the benchmarked output, kept for the whole-batch oracle check of the CPU leg
    gpu_out = (o.float().cpu().numpy(), sf.cpu().numpy()) if not args.no_cpu_baseline else None

    if not args.no_configs:
        csteps, cwarm = max(args.steps, 20), max(args.warmup, 20)
        result["configs"] = {
            "layer_340m": config_leg(torch, comba, dev, "layer_340m", csteps, cwarm, copies=3),
            "varlen": config_leg(torch, comba, dev, "varlen", csteps, cwarm, copies=2),
        }

    if not args.no_decode:
        wd = WORKLOADS["decode"]
        dec_copies = []
        for c in range(2):  # two resident copies so the 256 MB last-level cache cannot serve the state
            di = make_inputs(wd, seed=wd.seed + c)
            dec_copies.append(device_inputs(di, torch, dev))
        od = torch.empty((wd.B, 1, wd.H, wd.V), dtype=torch.bfloat16, device=dev)

        def dstep(i):
            c = dec_copies[i % 2]
            comba.recurrent_step(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["d"], c["s0"],
                                 in_place=True, out=od)

        dms, _ = time_loop(torch, dstep, max(args.steps, 20), args.warmup)
        ht = wd.B * wd.H
        dbytes = 2 * ht * wd.V * wd.K * 4 + ht * (2 * wd.K * 2 + 2 * wd.V * 2 + 8)
        result["decode"] = {"workload": "decode", "B": wd.B, "H": wd.H, "K": wd.K, "V": wd.V,
                            "us_per_step": dms * 1e3, "GB/s": dbytes / (dms * 1e-3) / 1e9,
                            "hbm_frac": dbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                            "algorithmic_bytes": dbytes, "kernel": "recurrent_kernel<128,128,32,bf16,bf16>",
                            "traffic": measured_traffic(kernel_source_hash(DECODE_SOURCES), DECODE_COUNTERS_JSON),
                            "step_us": step_distribution(torch, dstep)}
        if "measured_peaks" in result:
            result["decode"]["frac_of_measured_inplace"] = (dbytes / (dms * 1e-3) / 1e9
                                                            / result["measured_peaks"]["hbm_inplace_GB/s"])

    if not args.no_fused:
        raw = make_inputs(w, raw=True)
        tr = device_inputs(raw, torch, dev)

        def fstep(_):
            comba.chunk_fwd(tr["q"], tr["k"], tr["v"], tr["alpha"], tr["beta"], tr["d"], tr["s0"], out=o,
                            final_state=sf, gate_logits=True, qk_l2norm=True)

        fms, _ = time_loop(torch, fstep, args.steps, args.warmup)

        def split_step(_):
            # the same input steps as separate torch ops (bf16 q/k written back), then the unfused call
            qn = torch.nn.functional.normalize(tr["q"].float(), dim=-1, eps=1e-3).to(torch.bfloat16)
            kn = torch.nn.functional.normalize(tr["k"].float(), dim=-1, eps=1e-3).to(torch.bfloat16)
            comba.chunk_fwd(qn, kn, tr["v"], torch.sigmoid(tr["alpha"]), torch.sigmoid(tr["beta"]), tr["d"],
                            tr["s0"], out=o, final_state=sf)

        sms, _ = time_loop(torch, split_step, max(args.steps // 4, 10), min(args.warmup, 20))
        result["fused"] = {"workload": "layer_1p3b, raw q/k and gate logits", "flags": "gate_logits|qk_l2norm",
                           "us_per_step": fms * 1e3, "tokens/s": B * T / (fms * 1e-3),
                           "hbm_frac": nbytes / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "torch_preprocess_then_chunk_us": sms * 1e3}
        del tr

    if not args.no_shared_qk:
        # multi-value heads: one q / k head shared by the 16 value heads
        si = make_inputs(w, qk_heads=1)
        ts = device_inputs(si, torch, dev)

        def sstep(_):
            comba.chunk_fwd(ts["q"], ts["k"], ts["v"], ts["alpha"], ts["beta"], ts["d"], ts["s0"], out=o,
                            final_state=sf)

        qms, _ = time_loop(torch, sstep, max(args.steps // 2, 10), min(args.warmup, 50))
        sbytes = nbytes - B * T * H * 2 * K * 2 * (H - 1) // H  # q, k read once per shared head
        result["shared_qk"] = {"workload": "layer_1p3b with 1 q/k head for 16 value heads", "num_qk_heads": 1,
                               "us_per_step": qms * 1e3, "tokens/s": B * T / (qms * 1e-3),
                               "algorithmic_bytes": sbytes, "hbm_frac": sbytes / (qms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del ts, si

    if not args.no_backward:
        # training path: gradients of the same layer for seeded cotangents
        g = torch.Generator(device=dev)
        g.manual_seed(1234)
        do_ = torch.randn((B, T, H, V), generator=g, device=dev).to(torch.bfloat16)
        dsf_ = torch.randn((B, H, V, K), generator=g, device=dev)
        bws = torch.empty((comba.bwd_workspace_size(B, T, H, K, V),), dtype=torch.uint8, device=dev)

        def bstep(_):
            comba.chunk_bwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], do_, t["s0"], None, dsf_,
                            workspace=bws)

        bms, _ = time_loop(torch, bstep, max(args.steps // 10, 5), 5)
        # a training step: the forward, then the backward; either the backward
        # recomputes the chunk states, or the forward keeps them for it
        cs = torch.empty((comba.chunk_states_size(B, T, H, K, V) // 4,), dtype=torch.float32, device=dev)

        def train_recompute(_):
            step(0)
            bstep(0)

        def train_cached(_):
            comba.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], t["s0"], out=o, final_state=sf,
                            chunk_states=cs)
            comba.chunk_bwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], do_, t["s0"], None, dsf_,
                            workspace=bws, chunk_states=cs)

        trms, _ = time_loop(torch, train_recompute, max(args.steps // 10, 5), 5)
        tcms, _ = time_loop(torch, train_cached, max(args.steps // 10, 5), 5)
        del cs
        bbytes, bflops = chunk_bwd_algorithmic(B, T, H, K, V)
        result["backward"] = {"workload": "layer_1p3b, chunk backward (dq, dk, dv, dalpha, dbeta, dd, dS0)",
                              "us_per_step": bms * 1e3, "tokens/s": B * T / (bms * 1e-3),
                              "algorithmic_bytes": bbytes, "hbm_frac": bbytes / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                              "algorithmic_flops": bflops,
                              "train_step_us": {"forward_then_backward_recomputing_states": trms * 1e3,
                                                "forward_keeping_states_then_cached_backward": tcms * 1e3},
                              "mfma_frac": bflops / (bms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                              "workspace_bytes": bws.numel()}
        del bws, do_, dsf_

    if not args.no_long:
        # one 64K-token sequence: 32 workgroups plain, segment-parallel fills the chip
        wl_ = WORKLOADS["long_context"]
        li = make_inputs(wl_)
        tl = device_inputs(li, torch, dev)
        lo = torch.empty((1, wl_.T, wl_.H, wl_.V), dtype=torch.bfloat16, device=dev)
        lsf = torch.empty((1, wl_.H, wl_.V, wl_.K), dtype=torch.float32, device=dev)
        nws = comba.segmented_workspace_size(1, wl_.T, wl_.H, wl_.K, wl_.V, 0)
        lws = torch.empty((max(nws, 1),), dtype=torch.uint8, device=dev)

        def lstep(seg):
            return lambda _: comba.chunk_fwd(tl["q"], tl["k"], tl["v"], tl["alpha"], tl["beta"], tl["d"], None,
                                             out=lo, final_state=lsf, workspace=lws, segments=seg)

        lsteps, lwarm = max(args.steps // 10, 5), min(args.warmup // 10 + 2, 12)
        pms, _ = time_loop(torch, lstep(None), lsteps, lwarm)
        sms_, _ = time_loop(torch, lstep(0), lsteps, lwarm)
        lbytes, _ = chunk_fwd_algorithmic(1, wl_.T, wl_.H, wl_.K, wl_.V)
        result["long_context"] = {"workload": "long_context", "B": 1, "T": wl_.T, "H": wl_.H, "K": wl_.K, "V": wl_.V,
                                  "plain_us": pms * 1e3, "segmented_us": sms_ * 1e3,
                                  "segmented_tokens/s": wl_.T / (sms_ * 1e-3), "plain_tokens/s": wl_.T / (pms * 1e-3),
                                  "algorithmic_bytes": lbytes,
                                  "segmented_hbm_frac": lbytes / (sms_ * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                  "segments": "automatic (8 x 8192 tokens)", "workspace_bytes": nws}
        del tl, li

    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity"] = cpu_baseline(inp, H, gpu_out)

    if args.calibrate_copy:
        calibration_copy(torch, dev)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
