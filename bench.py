#!/usr/bin/env python3
"""Benchmark of the MSA forward pass on one MI355X.

One step = one msa_forward over the whole workload (index branch, inversion,
KV-outer sparse attention, combine; by default the last three once per pass of
16,384 query rows) with every input already resident in HBM.
Default workload: the 128K prefill with 64 planted hot blocks (N = 131,072,
H_q = 64, H_kv = 4, d_h = d_idx = 128, B_k = 128, k = 16, bf16), synthetic
seeded inputs.

Prints one JSON line: whole-job tokens/s, the sparse-counted TFLOP/s, per-kernel
times measured with HIP events on the launch stream, each kernel's roofline
fraction against the published peaks and against peaks measured on this GPU by
a probe for the same access patterns, the dense causal GQA kernel on the same
Q, K, V (the baseline MSA's speedup is quoted against), one decode step over 8
caches of the workload's shape, the training backward (msa_backward) on the
forward just timed, the same measurements of the forward for the 128K workload
with fp8 Q/K/V (`fp8`) and the 1M-token workload in 32K-row chunks
(`long_context`), and the CPU oracle timed on a bounded sample of the same
workload plus over every row of the tiny and 16K workloads.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# Sources whose change invalidates a recorded hardware-counter traffic figure
# of the attention kernel (its own code and the schedule it walks).
TRAFFIC_SOURCES = ("sparse_attn.hip", "msa_internal.h", "invert.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def sources_sha256() -> str:
    import hashlib
    hsh = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_attention_idx_amd", "csrc", name), "rb") as f:
            hsh.update(f.read())
    return hsh.hexdigest()


def recorded_traffic(workload: str, rows_per_launch: int):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary for this workload (FETCH_SIZE and WRITE_SIZE scaled by a plain
    copy of known size), or None when there is none, the kernel sources
    changed since the counters were taken, or they were taken with another
    number of query rows per launch."""
    path = os.path.join(ROOT, "profiles", f"sparse_attn_fwd_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            key, val = line[2:].split(":", 1)
            fields[key.strip()] = val.strip().strip("`")
    if fields.get("source_sha256") != sources_sha256():
        return None
    if fields.get("rows_per_launch") != str(rows_per_launch):
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measured_peaks():
    """Run the measured-peaks probe (a separate program built next to the
    library) and return its figures, or None when it is not built or fails."""
    import subprocess
    exe = os.path.join(ROOT, "block_sparse_attention_idx_amd", "msa_peaks")
    if not os.path.exists(exe):
        log("measured peaks: probe not built (block_sparse_attention_idx_amd.build.build_peaks)")
        return None
    log("measured peaks: running the probe")
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=180)
    except subprocess.TimeoutExpired:
        log("measured peaks: probe timed out")
        return None
    if r.returncode != 0:
        log(f"measured peaks: probe failed ({r.returncode}): {r.stderr.strip()[-300:]}")
        return None
    try:
        return json.loads(r.stdout.strip().splitlines()[-1])
    except (ValueError, IndexError):
        log("measured peaks: unreadable probe output")
        return None


# The measured peak each kernel is compared with: the indexer with sustained
# MFMA throughput on random operands (real Q and K tiles change from one MFMA
# to the next; the fixed-pattern figure, mfma_bf16_TFLOPs, runs at a higher
# clock), the attention kernel with the random 4 KB read/write mix (its Q
# gathers and partial-output stores), the combine with sequential reads (its
# partial slabs), the inversion with a plain copy.
MFMA_PEAK_KEY = "mfma_bf16_random_TFLOPs"
MEASURED_PEAK_OF = {"index_topk": MFMA_PEAK_KEY, "invert_blocks": "hbm_copy_GBs",
                    "sparse_attn_fwd": "hbm_rand4k_mixed_GBs", "combine": "hbm_seq_read_GBs"}


def path_accounting(acc, synth, w, sel):
    """Work of one forward from the selection it made (sel [batch * H_kv, N, k]):
    index and main-branch FLOPs and each kernel's algorithmic bytes -- the
    inversion reads and writes 4 B per slot, the attention writes the partials
    and reads each entry, Q once and K, V once per selected (group, block), the
    combine reads the partials and the selection and writes O."""
    f_idx = acc.index_flops(0, w.N, w.H_kv, w.d_idx, w.B_k, batch=w.batch)
    f_main = acc.main_flops(sel, 0, w.N, w.B_k, w.G, w.d_h)
    valid_slots = int((sel >= 0).sum())
    seq = np.arange(sel.shape[0], dtype=np.int64)[:, None, None]
    bins = int(np.count_nonzero(np.bincount((seq * w.B + sel)[sel >= 0], minlength=sel.shape[0] * w.B)))
    eb = 1 if w.dtype == "fp8" else 2
    part = acc.partial_bytes(valid_slots, w.G, w.d_h)
    return {
        "f_idx": f_idx, "f_main": f_main, "valid_slots": valid_slots,
        "attn": (part + 4 * valid_slots + w.batch * w.N * w.H_q * w.d_h * eb
                 + bins * 2 * w.B_k * w.d_h * eb),
        "comb": part + 4 * w.batch * w.H_kv * w.N * w.k + w.batch * w.N * w.H_q * w.d_h * 2,
        "inv": 4 * w.batch * w.H_kv * w.N * w.k + 4 * valid_slots,
    }


def kernel_table(kern, a):
    """Per-kernel time, algorithmic work and fraction of the published peak."""
    kernels = {
        "index_topk": {"ms": kern["index_topk"], "bound": "mfma", "flops": a["f_idx"],
                       "achieved": a["f_idx"] / kern["index_topk"] / 1e9, "peak": PEAK_BF16_TFLOPS,
                       "unit": "TFLOP/s"},
        "invert_blocks": {"ms": kern["invert_blocks"], "bound": "hbm", "bytes": a["inv"],
                          "achieved": a["inv"] / kern["invert_blocks"] / 1e6,
                          "peak": PEAK_HBM_GBS, "unit": "GB/s"},
        "sparse_attn_fwd": {"ms": kern["sparse_attn_fwd"], "bound": "hbm", "bytes": a["attn"],
                            "achieved": a["attn"] / kern["sparse_attn_fwd"] / 1e6,
                            "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "mfma_tflops": a["f_main"] / kern["sparse_attn_fwd"] / 1e9},
        "combine": {"ms": kern["combine"], "bound": "hbm", "bytes": a["comb"],
                    "achieved": a["comb"] / kern["combine"] / 1e6, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s"},
    }
    for v in kernels.values():
        v["frac"] = v["achieved"] / v["peak"]
    return kernels


def time_forward(msa, torch, fwd, steps, warmup, stream):
    """Mean, median and minimum ms of `steps` calls after `warmup` calls, from
    events recorded between consecutive calls on the launch stream."""
    for _ in range(warmup):
        fwd()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for j in range(steps):
        fwd()
        evs[j + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(evs[j].elapsed_time(evs[j + 1]) for j in range(steps))
    return evs[0].elapsed_time(evs[-1]) / steps, float(np.median(per)), per[0]


def rows_per_pass(msa, w):
    """The query rows msa_forward processes per pass for this workload: its
    q_chunk, or the library's default when that is 0."""
    qc = w.q_chunk if w.q_chunk else msa.DEFAULT_Q_CHUNK
    return min(qc, w.N)


def launches_per_step(kernel: str, w, qc: int) -> int:
    """Launches of a kernel in one msa_forward: the index branch runs once
    over all rows, the inversion, attention and combine once per pass."""
    return 1 if kernel == "index_topk" else -(-w.N // qc)


def time_chunked_kernels(msa, torch, d, o, t, w, bi_all, out, stream, dev, reps=1):
    """Per-kernel times of the chunked forward, summed over its chunks: the
    index branch once over all rows, then per chunk of q_chunk rows the chunk's
    selection rows copied out, the inversion, the attention and the combine,
    each bracketed by events on the launch stream (the steps msa_forward runs,
    through the entry points)."""
    qc = rows_per_pass(msa, w)
    seqs = w.batch * w.H_kv
    bi_c = torch.empty((w.batch, w.H_kv, qc, w.k), dtype=torch.int32, device=dev)
    sb = max(msa.msa_invert_workspace_size(d, qb, min(qc, w.N - qb)) for qb in range(0, w.N, qc))
    sched = torch.empty(((sb + 3) // 4,), dtype=torch.int32, device=dev)
    offs = torch.empty((seqs * (w.B + 1),), dtype=torch.int32, device=dev)
    ents = torch.empty((seqs * qc * w.k,), dtype=torch.int32, device=dev)
    opart = torch.empty((seqs * qc * w.k * w.G * w.d_h,), dtype=torch.bfloat16, device=dev)
    lpart = torch.empty((seqs * qc * w.k * w.G,), dtype=torch.float32, device=dev)
    tot = {"index_topk": 0.0, "invert_blocks": 0.0, "sparse_attn_fwd": 0.0, "combine": 0.0}
    for it in range(reps + 1):                 # pass 0 is a warmup
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        msa.msa_index_topk(d, t["q_idx"], t["k_idx"], block_idx=bi_all)
        e1.record(stream)
        marks = []
        for qb in range(0, w.N, qc):
            qn = min(qc, w.N - qb)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            sel = bi_c[:, :, :qn]
            sel.copy_(bi_all[:, :, qb:qb + qn])
            ev[0].record(stream)
            msa.msa_invert_blocks(d, sel, qb, qn, blk_offsets=offs, blk_entries=ents, sched=sched)
            ev[1].record(stream)
            msa.msa_sparse_attn_fwd(d, o, t["q"], t["k"], t["v"], offs, ents, sched, qb, qn,
                                    o_part=opart, lse_part=lpart)
            ev[2].record(stream)
            msa.msa_combine(d, sel, opart, lpart, qb, qn, o=out)
            ev[3].record(stream)
            marks.append(ev)
        torch.cuda.synchronize()
        if it == 0:
            continue
        tot["index_topk"] += e0.elapsed_time(e1) / reps
        for ev in marks:
            tot["invert_blocks"] += ev[0].elapsed_time(ev[1]) / reps
            tot["sparse_attn_fwd"] += ev[1].elapsed_time(ev[2]) / reps
            tot["combine"] += ev[2].elapsed_time(ev[3]) / reps
    return tot


def time_dense_in_ranges(msa, torch, d, o, t, w, out, stream, rows=16384):
    """The dense causal GQA kernel over every query row of the workload, one
    launch per range of `rows` queries (each launch well under a second), timed
    as one pass with events on the launch stream."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for qb in range(0, w.N, rows):
        msa.msa_dense_attn_fwd(d, o, t["q"], t["k"], t["v"], q_begin=qb, q_count=min(rows, w.N - qb), o=out)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def measure_workload(msa, acc, synth, torch, w, steps, warmup, dev, dense=False):
    """One more workload of the path, measured like the headline one: the
    whole msa_forward (inputs resident in HBM), each kernel's time (the four
    entry points, or the chunk loop through them), the work from the selection
    made, and the dominant kernel's roofline; with `dense`, also the dense
    causal GQA baseline over every row of the workload."""
    log(f"{w.name}: generating inputs on the device")
    stream = torch.cuda.current_stream(dev)
    t = {x: synth.device_tensor(w, x, dev) for x in ("q", "k", "v", "q_idx", "k_idx")}
    d = msa.make_dims(w.batch, w.N, w.H_q, w.H_kv, w.d_h, w.d_idx, w.B_k, w.k)
    s = synth.fp8_scale() if w.dtype == "fp8" else 1.0
    o = msa.make_opts(w.dtype, q_scale=s, k_scale=s, v_scale=s, q_chunk=w.q_chunk)
    out = torch.empty((w.batch, w.N, w.H_q, w.d_h), dtype=torch.bfloat16, device=dev)
    bi = torch.empty((w.batch, w.H_kv, w.N, w.k), dtype=torch.int32, device=dev)
    ws = torch.empty((msa.msa_workspace_size(d, o),), dtype=torch.uint8, device=dev)
    fwd = lambda: msa.msa_forward(d, o, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], o=out,
                                  block_idx_out=bi, workspace=ws)
    ms, med, mn = time_forward(msa, torch, fwd, steps, warmup, stream)
    log(f"{w.name}: msa_forward {ms:.3f} ms/step (median {med:.3f}, min {mn:.3f})")
    del ws
    torch.cuda.empty_cache()
    qc = rows_per_pass(msa, w)
    if qc < w.N:
        kern = time_chunked_kernels(msa, torch, d, o, t, w, bi, out, stream, dev)
    else:
        sb = msa.msa_invert_workspace_size(d, 0, w.N)
        sched = torch.empty(((sb + 3) // 4,), dtype=torch.int32, device=dev)
        offs = torch.empty((w.batch, w.H_kv, w.B + 1), dtype=torch.int32, device=dev)
        ents = torch.empty((w.batch * w.H_kv * w.N * w.k,), dtype=torch.int32, device=dev)
        opart = torch.empty((w.batch, w.H_kv, w.N, w.k, w.G, w.d_h), dtype=torch.bfloat16, device=dev)
        lpart = torch.empty((w.batch, w.H_kv, w.N, w.k, w.G), dtype=torch.float32, device=dev)
        names = ("index_topk", "invert_blocks", "sparse_attn_fwd", "combine")
        kern = dict.fromkeys(names, 0.0)
        for it in range(steps + 1):           # pass 0 is a warmup
            e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            e[0].record(stream)
            msa.msa_index_topk(d, t["q_idx"], t["k_idx"], block_idx=bi)
            e[1].record(stream)
            msa.msa_invert_blocks(d, bi, blk_offsets=offs, blk_entries=ents, sched=sched)
            e[2].record(stream)
            msa.msa_sparse_attn_fwd(d, o, t["q"], t["k"], t["v"], offs, ents, sched,
                                    o_part=opart, lse_part=lpart)
            e[3].record(stream)
            msa.msa_combine(d, bi, opart, lpart, o=out)
            e[4].record(stream)
            torch.cuda.synchronize()
            if it:
                for j, name in enumerate(names):
                    kern[name] += e[j].elapsed_time(e[j + 1]) / steps
    log(f"{w.name}: per kernel ms: " + ", ".join(f"{k} {v:.3f}" for k, v in kern.items()))
    dense_res = None
    if dense:
        # a short warm launch first (the last 256 rows), then every row once
        msa.msa_dense_attn_fwd(d, o, t["q"], t["k"], t["v"], q_begin=w.N - 256, q_count=256, o=out)
        torch.cuda.synchronize()
        log(f"{w.name}: dense baseline over all {w.N} rows in 16,384-row launches")
        dms = time_dense_in_ranges(msa, torch, d, o, t, w, out, stream)
        f_dense = acc.dense_flops(0, w.N, w.H_q, w.d_h, batch=w.batch)
        dense_res = {"kernel": "dense_attn_fwd", "ms": dms, "bound": "mfma", "flops": f_dense,
                     "achieved": f_dense / dms / 1e9, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": f_dense / dms / 1e9 / PEAK_BF16_TFLOPS,
                     "tokens_s": w.batch * w.N / (dms * 1e-3), "msa_speedup": dms / ms,
                     "launches": -(-w.N // 16384)}
        log(f"{w.name}: dense baseline {dms:.1f} ms, {dense_res['achieved']:.0f} TFLOP/s; "
            f"msa_forward is {dense_res['msa_speedup']:.2f}x faster")
    sel = bi.cpu().numpy().reshape(w.batch * w.H_kv, w.N, w.k)
    del t, out, bi
    torch.cuda.empty_cache()
    a = path_accounting(acc, synth, w, sel)
    kernels = kernel_table(kern, a)
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    dk = kernels[dom]
    traffic = recorded_traffic(w.name, qc) if dom == "sparse_attn_fwd" else None
    launches = launches_per_step(dom, w, qc)
    roofline = {"kernel": dom, "bound": dk["bound"], "achieved": dk["achieved"], "peak": dk["peak"],
                "unit": dk["unit"], "frac": dk["frac"], "traffic": traffic,
                "launches_per_step": launches, "ms_per_launch": dk["ms"] / launches}
    if traffic:
        roofline["traffic_achieved"] = traffic * launches / dk["ms"] / 1e6
    return {
        "workload": w.name, "dtype": w.dtype, "N": w.N, "q_chunk": qc, "steps": steps,
        "warmup": warmup, "ms_per_step": ms, "ms_median": med, "ms_min": mn,
        "tokens_s": w.batch * w.N / (ms * 1e-3),
        "sparse_tflops": (a["f_idx"] + a["f_main"]) / (ms * 1e-3) / 1e12,
        "index_flops": a["f_idx"], "main_flops": a["f_main"],
        "roofline": roofline,
        "kernels": kernels,
        "dense_baseline": dense_res,
    }


def cpu_full_run(oracle, synth, acc, w):
    """The oracle over every row of a workload (index branch, then the main
    branch on its selection), timed on this host."""
    rows = np.arange(w.N)
    qi = synth.host_rows(w, "q_idx", rows)
    ki = synth.host_all(w, "k_idx")
    qr = synth.host_rows(w, "q", rows)
    K = synth.host_all(w, "k")
    V = synth.host_all(w, "v")
    c0 = time.perf_counter()
    obi, _, _ = oracle.index_topk(w.N, w.B_k, w.k, rows, qi, ki)
    oracle.attention(w.N, w.B_k, rows, qr, K, V, obi)
    csec = time.perf_counter() - c0
    flops = acc.index_flops(0, w.N, w.H_kv, w.d_idx, w.B_k) + acc.main_flops(obi, 0, w.N, w.B_k, w.G, w.d_h)
    return {"workload": w.name, "rows": int(w.N), "seconds": csec, "value": w.N / csec,
            "unit": "tokens/s", "gflops": flops / csec / 1e9}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_n131072_hq64_hkv4_k16_hot64")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=3072,
                    help="query rows of the oracle sample (all heads and groups)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured-peaks probe (HBM patterns and MFMA throughput)")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense causal GQA baseline on the same Q, K, V")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode step (last token of 8 sequences of the workload's length)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the selection-variant timings (block sizes, index heads, forced and "
                         "sliding-window selections)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the training backward pass (msa_backward) timing")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the 128K forward with fp8 Q/K/V")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the 1M-token forward in 32K-row chunks")
    ap.add_argument("--no-cpu-full", action="store_true",
                    help="skip the oracle over every row of the tiny and 16K workloads")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB (a kernel "
                         "of known traffic, to calibrate hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the MSA forward path here is a single-GPU "
              "build (no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_attention_idx_amd as msa
    from block_sparse_attention_idx_amd import accounting as acc
    import synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy_mib > 0:
        src = torch.ones(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB written")
        del src, dst
    log(f"workload {w.name}: generating inputs on the device")
    t = {x: synth.device_tensor(w, x, dev) for x in ("q", "k", "v", "q_idx", "k_idx")}
    d = msa.make_dims(w.batch, w.N, w.H_q, w.H_kv, w.d_h, w.d_idx, w.B_k, w.k)
    if w.dtype == "fp8":
        s = synth.fp8_scale()
        o = msa.make_opts("fp8", q_scale=s, k_scale=s, v_scale=s, q_chunk=w.q_chunk)
    else:
        o = msa.make_opts("bf16", q_chunk=w.q_chunk)
    out = torch.empty((w.batch, w.N, w.H_q, w.d_h), dtype=torch.bfloat16, device=dev)
    bi = torch.empty((w.batch, w.H_kv, w.N, w.k), dtype=torch.int32, device=dev)
    ws = torch.empty((msa.msa_workspace_size(d, o),), dtype=torch.uint8, device=dev)
    args_f = (d, o, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"])
    stream = torch.cuda.current_stream(dev)

    # ---- whole-step timing: msa_forward
    log(f"warmup {args.warmup}, timed steps {args.steps}")
    for _ in range(args.warmup):
        msa.msa_forward(*args_f, o=out, block_idx_out=bi, workspace=ws)
    torch.cuda.synchronize()
    # an event between consecutive steps gives the per-step times as well
    evs_f = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs_f[0].record(stream)
    for j in range(args.steps):
        msa.msa_forward(*args_f, o=out, block_idx_out=bi, workspace=ws)
        evs_f[j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = evs_f[0].elapsed_time(evs_f[-1]) / args.steps
    step_ms = sorted(evs_f[j].elapsed_time(evs_f[j + 1]) for j in range(args.steps))
    ms_median, ms_min = float(np.median(step_ms)), step_ms[0]
    log(f"msa_forward: {ms_step:.3f} ms/step (median {ms_median:.3f}, min {ms_min:.3f}; "
        f"host wall {1e3 * wall / args.steps:.3f} ms/step)")

    # ---- per-kernel timing: the same pass through the four entry points, with
    # HIP events between the calls on the launch stream (chunked: the chunk
    # loop msa_forward runs, summed over the chunks)
    kern = {}
    qc = rows_per_pass(msa, w)
    lse_out = torch.empty((w.batch, w.N, w.H_q), dtype=torch.float32, device=dev)
    opart = lpart = None
    if qc < w.N:
        kern = time_chunked_kernels(msa, torch, d, o, t, w, bi, out, stream, dev, reps=args.steps)
        log("per call ms (summed over the chunks): " + ", ".join(f"{k} {v:.3f}" for k, v in kern.items()))
        # the output and LSE the backward starts from
        msa.msa_forward(*args_f, o=out, lse=lse_out, block_idx_out=bi, workspace=ws)
        torch.cuda.synchronize()
        del ws
        torch.cuda.empty_cache()
    else:
        sb = msa.msa_invert_workspace_size(d, 0, w.N)
        sched = torch.empty(((sb + 3) // 4,), dtype=torch.int32, device=dev)
        offs = torch.empty((w.batch, w.H_kv, w.B + 1), dtype=torch.int32, device=dev)
        ents = torch.empty((w.batch * w.H_kv * w.N * w.k,), dtype=torch.int32, device=dev)
        opart = torch.empty((w.batch, w.H_kv, w.N, w.k, w.G, w.d_h), dtype=torch.bfloat16, device=dev)
        lpart = torch.empty((w.batch, w.H_kv, w.N, w.k, w.G), dtype=torch.float32, device=dev)
        del ws
        torch.cuda.empty_cache()
        names = ("index_topk", "invert_blocks", "sparse_attn_fwd", "combine")
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps + 1)]
        for it in range(args.steps + 1):       # iteration 0 is a warmup
            e = evs[it]
            e[0].record(stream)
            msa.msa_index_topk(d, t["q_idx"], t["k_idx"], block_idx=bi)
            e[1].record(stream)
            msa.msa_invert_blocks(d, bi, blk_offsets=offs, blk_entries=ents, sched=sched)
            e[2].record(stream)
            msa.msa_sparse_attn_fwd(d, o, t["q"], t["k"], t["v"], offs, ents, sched,
                                    o_part=opart, lse_part=lpart)
            e[3].record(stream)
            msa.msa_combine(d, bi, opart, lpart, o=out, lse=lse_out)
            e[4].record(stream)
        torch.cuda.synchronize()
        for j, name in enumerate(names):
            kern[name] = float(np.mean([evs[it][j].elapsed_time(evs[it][j + 1])
                                        for it in range(1, args.steps + 1)]))
        log("per call ms: " + ", ".join(f"{k} {v:.3f}" for k, v in kern.items()))

    # ---- the training backward (msa_backward: main-branch dQ, dK, dV and the
    # KL alignment gradient of the index branch) on the forward just timed,
    # for single-chunk bf16 workloads; dO is seeded N(0, 1)
    backward = None
    if kern and not args.no_backward and w.dtype == "bf16":
        opart = lpart = None
        torch.cuda.empty_cache()
        d_o = synth.device_tensor(w, "d_o", dev)
        wsb = torch.empty((msa.msa_backward_workspace_size(d, o),), dtype=torch.uint8, device=dev)
        bargs = (d, o, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], out, lse_out, d_o, bi)
        kw = 1.0 / (w.batch * w.N * w.H_sel)
        log("backward: 1 warmup, 3 timed calls")
        msa.msa_backward(*bargs, kl_weight=kw, workspace=wsb)
        torch.cuda.synchronize()
        eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        eb0.record(stream)
        for _ in range(3):
            msa.msa_backward(*bargs, kl_weight=kw, workspace=wsb)
        eb1.record(stream)
        torch.cuda.synchronize()
        bms = eb0.elapsed_time(eb1) / 3
        sel_b = bi.cpu().numpy().reshape(w.batch * w.H_sel, w.N, w.k)
        fb_main, fb_idx = acc.backward_flops(sel_b, 0, w.N, w.B_k, w.G_sel, w.d_h, w.d_idx)
        backward = {"call": "msa_backward", "ms": bms, "bound": "mfma", "flops_main": fb_main,
                    "flops_index": fb_idx, "achieved": (fb_main + fb_idx) / bms / 1e9,
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": (fb_main + fb_idx) / bms / 1e9 / PEAK_BF16_TFLOPS,
                    "tokens_s": w.batch * w.N / (bms * 1e-3), "workspace_bytes": wsb.numel()}
        log(f"backward: {bms:.2f} ms, {backward['achieved']:.0f} TFLOP/s")
        del d_o, wsb
        torch.cuda.empty_cache()

    # ---- selection variants (the paper's ablations) on the same Q, K, V,
    # Q^idx, K^idx: 64- and 32-token key blocks (k = 32), eight index heads
    # over the four K/V heads, the forced first block with a 4-block local
    # window, and the FLOP-matched sliding window; each is one whole pass
    # (selection, inversion, attention, combine) timed like the forward
    variants = None
    if kern and not args.no_variants and w.dtype == "bf16":
        variants = {}

        def timed(fn, reps=3):
            fn()
            torch.cuda.synchronize()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            for _ in range(reps):
                fn()
            a1.record(stream)
            torch.cuda.synchronize()
            return a0.elapsed_time(a1) / reps

        def record(name, dv, ms, biv):
            selv = biv.cpu().numpy().reshape(-1, w.N, dv.k)
            f_m = acc.main_flops(selv, 0, w.N, dv.B_k, w.H_q // dv.H_sel, w.d_h)
            f_i = acc.index_flops(0, w.N, dv.H_sel, w.d_idx, dv.B_k, batch=w.batch)
            variants[name] = {"ms": ms, "tokens_s": w.batch * w.N / (ms * 1e-3), "B_k": dv.B_k, "k": dv.k,
                              "H_idx": dv.H_sel, "index_flops": f_i, "main_flops": f_m,
                              "sparse_tflops": (f_i + f_m) / (ms * 1e-3) / 1e12}
            log(f"variant {name}: {ms:.2f} ms, {variants[name]['sparse_tflops']:.0f} sparse TFLOP/s")

        qi8 = synth.device_tensor(w.with_(H_idx=8), "q_idx", dev)
        for name, B_k, k, H_idx, qiv in (("block64_k32", 64, 32, 0, t["q_idx"]),
                                         ("block32_k32", 32, 32, 0, t["q_idx"]),
                                         ("index_heads8", w.B_k, w.k, 8, qi8)):
            dv = msa.make_dims(w.batch, w.N, w.H_q, w.H_kv, w.d_h, w.d_idx, B_k, k, H_idx=H_idx)
            biv = torch.empty((w.batch, dv.H_sel, w.N, k), dtype=torch.int32, device=dev)
            wsv = torch.empty((msa.msa_workspace_size(dv, o),), dtype=torch.uint8, device=dev)
            ms = timed(lambda: msa.msa_forward(dv, o, t["q"], t["k"], t["v"], qiv, t["k_idx"], o=out,
                                               block_idx_out=biv, workspace=wsv))
            record(name, dv, ms, biv)
            del biv, wsv
            torch.cuda.empty_cache()
        del qi8

        # composed passes: the selection call, then the inversion, attention
        # and combine entry points on preallocated buffers
        sb_v = msa.msa_invert_workspace_size(d, 0, w.N)
        sched_v = torch.empty(((sb_v + 3) // 4,), dtype=torch.int32, device=dev)
        offs_v = torch.empty((w.batch, w.H_kv, w.B + 1), dtype=torch.int32, device=dev)
        ents_v = torch.empty((w.batch * w.H_kv * w.N * w.k,), dtype=torch.int32, device=dev)
        op_v = torch.empty((w.batch, w.H_kv, w.N, w.k, w.G, w.d_h), dtype=torch.bfloat16, device=dev)
        lp_v = torch.empty((w.batch, w.H_kv, w.N, w.k, w.G), dtype=torch.float32, device=dev)
        biv = torch.empty((w.batch, w.H_kv, w.N, w.k), dtype=torch.int32, device=dev)

        def rest():
            msa.msa_invert_blocks(d, biv, blk_offsets=offs_v, blk_entries=ents_v, sched=sched_v)
            msa.msa_sparse_attn_fwd(d, o, t["q"], t["k"], t["v"], offs_v, ents_v, sched_v,
                                    o_part=op_v, lse_part=lp_v)
            msa.msa_combine(d, biv, op_v, lp_v, o=out)

        ms = timed(lambda: (msa.msa_index_topk_forced(d, t["q_idx"], t["k_idx"], force_first=True,
                                                       local_window=4, block_idx=biv), rest()))
        record("forced_first_window4", d, ms, biv)
        ms = timed(lambda: (msa.msa_window_select(d, block_idx=biv), rest()))
        record("sliding_window", d, ms, biv)
        del sched_v, offs_v, ents_v, op_v, lp_v, biv
        torch.cuda.empty_cache()

    # ---- the dense causal GQA baseline on the same Q, K, V (bf16 workloads up
    # to 128K tokens: it grows quadratically, 0.3 s per call at 128K)
    dense = None
    if not args.no_dense and w.dtype == "bf16" and w.batch * w.N <= 131072:
        log("dense baseline: 1 warmup, 3 timed calls")
        msa.msa_dense_attn_fwd(d, o, t["q"], t["k"], t["v"], o=out)
        ed0, ed1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ed0.record(stream)
        for _ in range(3):
            msa.msa_dense_attn_fwd(d, o, t["q"], t["k"], t["v"], o=out)
        ed1.record(stream)
        torch.cuda.synchronize()
        dms = ed0.elapsed_time(ed1) / 3
        f_dense = acc.dense_flops(0, w.N, w.H_q, w.d_h, batch=w.batch)
        dense = {"kernel": "dense_attn_fwd", "ms": dms, "bound": "mfma", "flops": f_dense,
                 "achieved": f_dense / dms / 1e9, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                 "frac": f_dense / dms / 1e9 / PEAK_BF16_TFLOPS,
                 "tokens_s": w.batch * w.N / (dms * 1e-3), "msa_speedup": dms / ms_step}
        log(f"dense baseline: {dms:.2f} ms, {dense['achieved']:.0f} TFLOP/s; "
            f"msa_forward is {dense['msa_speedup']:.2f}x faster")

    # ---- decode: one new token per sequence against caches of the workload's
    # shape (8 sequences up to 128K tokens, else 1), inputs resident in HBM
    decode = None
    if not args.no_decode and w.dtype == "bf16":
        nb_dec = 8 if w.N <= 131072 else 1
        wd = w.with_(batch=nb_dec, q_chunk=0)
        log(f"decode: {nb_dec} sequences of {wd.N} tokens: generating caches")
        last = np.arange(nb_dec) * wd.N + (wd.N - 1)
        qd = torch.from_numpy(synth.host_rows(wd, "q", last).view(np.int16)).to(dev).view(torch.bfloat16)
        qid = torch.from_numpy(synth.host_rows(wd, "q_idx", last).view(np.int16)).to(dev).view(torch.bfloat16)
        kd, vd, kid = (synth.device_tensor(wd, x, dev) for x in ("k", "v", "k_idx"))
        dd = msa.make_dims(wd.batch, wd.N, wd.H_q, wd.H_kv, wd.d_h, wd.d_idx, wd.B_k, wd.k)
        od = msa.make_opts("bf16")
        bid = torch.empty((wd.batch, wd.H_kv, wd.k), dtype=torch.int32, device=dev)
        wsd = torch.empty((msa.msa_decode_workspace_size(dd, od),), dtype=torch.uint8, device=dev)
        outd = torch.empty((wd.batch, wd.H_q, wd.d_h), dtype=torch.bfloat16, device=dev)
        dargs = (dd, od, qd, qid, kd, vd, kid)
        for _ in range(3):
            msa.msa_decode(*dargs, o=outd, block_idx_out=bid, workspace=wsd)
        torch.cuda.synchronize()
        reps = 50
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            msa.msa_decode(*dargs, o=outd, block_idx_out=bid, workspace=wsd)
        e1.record(stream)
        torch.cuda.synchronize()
        dec_ms = e0.elapsed_time(e1) / reps
        sel_d = bid.cpu().numpy()
        valid_d = int((sel_d >= 0).sum())
        L_d = (wd.N - 1) // wd.B_k
        b_dec = acc.decode_bytes(wd.batch, wd.N, wd.H_q, wd.H_kv, wd.d_h, wd.d_idx, wd.B_k, wd.k, valid_d)
        decode = {"batch": wd.batch, "context": wd.N, "ms": dec_ms, "tokens_s": wd.batch / (dec_ms * 1e-3),
                  "bound": "hbm", "bytes": b_dec, "achieved": b_dec / dec_ms / 1e6,
                  "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": b_dec / dec_ms / 1e6 / PEAK_HBM_GBS,
                  "index_scan_bytes": wd.batch * L_d * wd.B_k * wd.d_idx * 2}
        log(f"decode: {dec_ms * 1e3:.1f} us per step, {decode['achieved']:.0f} GB/s algorithmic")
        del qd, qid, kd, vd, kid, wsd, outd, bid
        torch.cuda.empty_cache()

    # ---- work accounting from the selection actually made
    sel = bi.cpu().numpy().reshape(w.batch * w.H_kv, w.N, w.k)
    acct = path_accounting(acc, synth, w, sel)
    f_idx, f_main = acct["f_idx"], acct["f_main"]
    # block popularity: non-local selections per (sequence, group, block), the
    # skew the pre-scheduled chunking absorbs
    loc = (np.arange(w.N) // w.B_k)[None, :, None]
    nonlocal_sel = (sel >= 0) & (sel != loc)
    counts = np.zeros((sel.shape[0], w.B), np.int64)
    for g in range(sel.shape[0]):
        counts[g] = np.bincount(sel[g][nonlocal_sel[g]], minlength=w.B)[:w.B]
    popularity = {"max": int(counts.max()), "mean": float(counts.mean()),
                  "p99": float(np.percentile(counts, 99)),
                  "max_over_mean": float(counts.max() / max(counts.mean(), 1e-9))}
    if w.plant:
        hot = np.zeros(w.B, bool)
        hot[synth.hot_blocks(w)] = True
        if hot.any() and (~hot).any():
            popularity["hot_mean"] = float(counts[:, hot].mean())
            popularity["other_mean"] = float(counts[:, ~hot].mean())
    tokens_s = w.batch * w.N / (ms_step * 1e-3)
    tflops = (f_idx + f_main) / (ms_step * 1e-3) / 1e12

    kernels = {}
    if kern:
        kernels = kernel_table(kern, acct)
        dom = max(kernels, key=lambda n: kernels[n]["ms"])
        dk = kernels[dom]
        traffic = recorded_traffic(w.name, qc) if dom == "sparse_attn_fwd" else None
        launches = launches_per_step(dom, w, qc)
        # a step launches the attention once per pass (the index branch once):
        # achieved is the step's algorithmic bytes (or FLOPs) over their summed
        # launch time, the same as per launch on average; traffic is per launch
        roofline = {"kernel": dom, "bound": dk["bound"], "achieved": dk["achieved"],
                    "peak": dk["peak"], "unit": dk["unit"], "frac": dk["frac"],
                    "traffic": traffic, "launches_per_step": launches,
                    "ms_per_launch": dk["ms"] / launches}
        if traffic:
            # the counted HBM bytes over the same launch time (GB/s)
            roofline["traffic_achieved"] = traffic * launches / dk["ms"] / 1e6
    else:
        roofline = None

    # ---- measured peaks of this GPU for the patterns the kernels use
    peaks = None if args.no_peaks else measured_peaks()
    if peaks:
        log("measured peaks: " + ", ".join(f"{k} {v}" for k, v in peaks.items()))
        for name, v in kernels.items():
            key = MEASURED_PEAK_OF.get(name)
            if key in peaks and peaks[key] > 0:
                v["measured_peak"] = peaks[key]
                v["measured_peak_kind"] = key
                v["frac_measured"] = v["achieved"] / peaks[key]
        if decode and peaks.get("hbm_seq_read_GBs", 0) > 0:
            decode["measured_peak"] = peaks["hbm_seq_read_GBs"]
            decode["measured_peak_kind"] = "hbm_seq_read_GBs"
            decode["frac_measured"] = decode["achieved"] / peaks["hbm_seq_read_GBs"]
        if dense and peaks.get(MFMA_PEAK_KEY, 0) > 0:
            dense["measured_peak"] = peaks[MFMA_PEAK_KEY]
            dense["measured_peak_kind"] = MFMA_PEAK_KEY
            dense["frac_measured"] = dense["achieved"] / peaks[MFMA_PEAK_KEY]
        if roofline and roofline.get("traffic_achieved") and roofline["kernel"] in kernels:
            mp = kernels[roofline["kernel"]].get("measured_peak")
            if mp:
                roofline["traffic_frac_measured"] = roofline["traffic_achieved"] / mp

    # ---- the other workloads of the path: the 128K forward with fp8 Q/K/V and
    # the 1M-token forward in 32K-row chunks (the headline workload's device
    # buffers are released first)
    del t, out, bi
    opart = lpart = sched = offs = ents = lse_out = None
    torch.cuda.empty_cache()
    fp8 = long_ctx = None
    if not args.no_fp8 and w.name != synth.P128K_FP8.name:
        fp8 = measure_workload(msa, acc, synth, torch, synth.P128K_FP8, args.steps, args.warmup, dev)
    if not args.no_long_context and w.name != synth.P1M.name:
        long_ctx = measure_workload(msa, acc, synth, torch, synth.P1M, 2, 1, dev, dense=not args.no_dense)

    # ---- the CPU oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        rng = np.random.default_rng(12345)
        rows = np.sort(rng.choice(w.N, size=min(args.cpu_rows, w.N), replace=False))
        log(f"cpu baseline: host inputs for {len(rows)} sampled rows")
        qi = synth.host_rows(w, "q_idx", rows)
        ki = synth.host_all(w, "k_idx")
        qr = synth.host_rows(w, "q", rows)
        K = synth.host_all(w, "k")
        V = synth.host_all(w, "v")
        code = oracle.FP8 if w.dtype == "fp8" else oracle.BF16
        sc = synth.fp8_scale() if w.dtype == "fp8" else 1.0
        oracle.lib()
        log("cpu baseline: timing the oracle")
        c0 = time.perf_counter()
        obi, _, _ = oracle.index_topk(w.N, w.B_k, w.k, rows, qi, ki)
        oracle.attention(w.N, w.B_k, rows, qr, K, V, obi, dtype=code, q_scale=sc, k_scale=sc,
                         v_scale=sc)
        csec = time.perf_counter() - c0
        sample_flops = (float((rows // w.B_k).sum()) * 2 * w.d_idx * w.H_kv * w.B_k
                        + acc.main_flops(obi, 0, w.N, w.B_k, w.G, w.d_h) / 1.0)
        model = None
        try:
            with open("/proc/cpuinfo") as f:
                model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
        except OSError:
            pass
        cpu = {"value": len(rows) / csec, "unit": "tokens/s", "cores": oracle.num_threads(),
               "cpu_model": model,
               "kind": "oracle", "seconds": csec, "gflops": sample_flops / csec / 1e9,
               "extrapolated_full_seconds": csec * (f_idx + f_main) / sample_flops,
               "sample": f"{len(rows)} seeded random query rows of {w.name}, all {w.H_kv} groups "
                         f"and {w.H_q} heads: index branch (fp32) + sparse attention (fp64)"}
        log(f"cpu baseline: {csec:.1f} s -> {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")
        if not args.no_cpu_full:
            # the oracle over every row of the tiny and the 16K workloads
            cpu["full_runs"] = {}
            for wf in (synth.TINY, synth.P16K):
                log(f"cpu baseline: the oracle over all {wf.N} rows of {wf.name}")
                r = cpu_full_run(oracle, synth, acc, wf)
                cpu["full_runs"][wf.name] = r
                log(f"cpu baseline: {r['seconds']:.1f} s -> {r['value']:.1f} tokens/s")

    line = {
        "metric": "MSA fwd sparse TFLOP/s + tokens/s at N=128K (Hq64/Hkv4/d128/k16); % MFMA/HBM peak",
        "value": tokens_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "N": w.N, "H_q": w.H_q, "H_kv": w.H_kv,
                   "d_h": w.d_h, "d_idx": w.d_idx, "B_k": w.B_k, "k": w.k,
                   "q_chunk": qc, "hot_blocks": w.plant},
        "ms_median": ms_median, "ms_min": ms_min,
        "sparse_tflops": tflops, "index_flops": f_idx, "main_flops": f_main,
        "block_popularity": popularity,
        "roofline": roofline, "kernels": kernels, "dense_baseline": dense, "decode": decode,
        "backward": backward, "variants": variants, "fp8": fp8, "long_context": long_ctx,
        "measured_peaks": peaks, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
