#!/usr/bin/env python3
"""MLA paged decode benchmark on one MI355X.

One step = one full decode of the batch through the C ABI (mla_decode): the
stream kernel (paged KV stream, Q.K^T, base-2 online softmax, P.V, partials
or finished rows) and the merge kernel (output + natural-log LSE, sinks).

Headline workload: bs=52 requests, qlen=1, 16 heads, 16384 KV tokens per
request, bf16 q and latent cache ~N(0,1), block 64 = TILE 64, random block
table permutation, scale 1/sqrt(192), balanced split.  The default run also
times every other benchmark configuration (16-head fp8, 48- and 64-head fp8,
128-head bf16 with 256-token blocks, the ragged 128-request causal batch)
under both schedules (the balanced split and the segment partition at the
planner's S) and appends them under "extra", each with its own roofline.
--extra adds the fused q prologue, the index streams and the DCP emulation.

Inputs are synthetic (seeded) and resident in HBM before timing starts; two
cache copies alternate between steps so no step reuses the previous step's
cache lines from the 256 MB last-level cache.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per MLA decode step and effective KV HBM GB/s (bs=52, 16K ctx, H=16..128)"
HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    # name: workload constructor (seeded; see mla_inputs)
    "bs52_ctx16k_h16_bf16_blk64": lambda mi: mi.bs52_h16_bf16(),
    "bs52_ctx16k_h16_fp8_blk64": lambda mi: mi.bs52_fp8(16),
    "bs52_ctx16k_h48_fp8_blk64": lambda mi: mi.bs52_fp8(48),
    "bs52_ctx16k_h64_fp8_blk64": lambda mi: mi.bs52_fp8(64),
    "bs52_ctx16k_h128_bf16_blk256": lambda mi: mi.bs52_h128_bf16(),
    "ragged128_max32k_h96_fp8_causal_sinks": lambda mi: mi.ragged_h96_fp8(),
    # the fused q prologue: bf16 q quantised to e4m3 in the q load
    "bs52_ctx16k_h48_fp8_blk64_bf16q": lambda mi: mi.with_bf16_q(mi.bs52_fp8(48), seed=3),
    # index-stream (sparse top-k) decode: page size 1, per-token index lists
    "sparse_bs52_top2048_ctx16k_h16_bf16": lambda mi: mi.sparse_bs52(16, "bf16"),
    "sparse_bs52_top2048_ctx16k_h128_fp8": lambda mi: mi.sparse_bs52(128, "fp8_e4m3"),
}
DEFAULT = "bs52_ctx16k_h16_bf16_blk64"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--extra", action="store_true",
                    help="also time the q prologue, index-stream and DCP workloads")
    ap.add_argument("--only", action="store_true", help="time the --workload alone (no other configurations)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-reqs", type=int, default=0, help="requests the oracle times (0 = all)")
    ap.add_argument("--schedule", default="balanced", choices=["balanced", "segments"],
                    help="schedule of the headline line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    return ap.parse_args()


def copy_calibration(torch, reps=5):
    """A plain copy of known size: the HBM counters read for it calibrate the
    segment kernel's FETCH_SIZE / WRITE_SIZE per launch."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "reps": reps}), flush=True)


def build_inputs(name, torch, mi):
    w = WORKLOADS[name](mi)
    w.name = name
    d = mi.to_torch(w, "cuda")
    # a second cache copy (same contents, other addresses) for alternating steps
    d2 = dict(d)
    d2["kv_cache"] = d["kv_cache"].clone()
    return w, [d, d2]


WARMUP_FLOOR_S = 0.3


def warmup(fn, n, torch):
    """n untimed calls, continued until WARMUP_FLOOR_S has passed: the GPU
    clocks take some tens of milliseconds to settle after the first launches,
    and a handful of 0.2 ms steps would otherwise be timed during that ramp."""
    t0 = time.perf_counter()
    i = 0
    while i < n or time.perf_counter() - t0 < WARMUP_FLOOR_S:
        fn(i)
        i += 1
        if i % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


DCP_WORKLOADS = {
    # decode context parallelism emulated on one GPU: (shards, base batch)
    "dcp4_bs52_ctx16k_h16_bf16_blk64": (4, lambda mi: mi.bs52_h16_bf16()),
}


def time_dcp(name, args, torch, m, mi):
    """One rank's share of a DCP step (its shard's decode + the LSE combine of
    every shard's output) and the whole step emulated on one GPU (every shard's
    decode, then the combine)."""
    W, ctor = DCP_WORKLOADS[name]
    w = ctor(mi)
    shards = mi.dcp_shards(w, W)
    ds = [mi.to_torch(sw, "cuda") for sw in shards]
    T, H = w.num_tokens, w.num_heads
    so = torch.empty((W, T, H, 512), dtype=torch.bfloat16, device="cuda")
    sl = torch.empty((W, T, H), dtype=torch.float32, device="cuda")
    # each shard decodes straight into its slice of the stacked buffers
    decs = [m.Decoder(**mi.call_args(sw, d), sinks=None, schedule="balanced", out=so[k], lse=sl[k])
            for k, (sw, d) in enumerate(zip(shards, ds))]
    sinks = torch.randn(H, generator=torch.Generator().manual_seed(11)).cuda()
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def combine():
        m.combine_lse(so, sl, sinks=sinks, out=out, lse=lse, stream=stream)

    def timed(fn):
        warmup(lambda i: fn(), args.warmup, torch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps * 1e3

    for dec in decs:
        dec.run(stream)
    t_rank_decode = timed(lambda: decs[0].run(stream))
    t_combine = timed(combine)
    t_step = timed(lambda: ([d.run(stream) for d in decs], combine()))
    kv_bytes = w.kv_bytes_touched()
    return {"workload": name, "num_shards": W, "num_heads": H, "dtype": w.kv_dtype,
            "num_reqs": w.num_reqs, "max_seq_len": w.max_seq_len,
            "shard_decode_us": round(t_rank_decode, 2), "combine_us": round(t_combine, 2),
            "rank_step_us": round(t_rank_decode + t_combine, 2),
            "emulated_step_us": round(t_step, 2),
            "eff_kv_GBps_emulated": kv_bytes / (t_step * 1e-6) / 1e9,
            "split_workgroups": decs[0].split_workgroups}


FP8_MFMA_PEAK_TFLOPS = 5000.0   # dense fp8 MFMA peak of MI355X
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16


def attention_flops(w):
    """MFMA work of one decode step: per (query row, visible key) 576 MACs of
    Q.K^T and 512 of P.V, 2 flops each."""
    qo = [int(x) for x in w.qo_indptr]
    rows_keys = 0
    for r, L in enumerate(int(x) for x in w.seq_lens):
        ql = qo[r + 1] - qo[r]
        for i in range(ql):
            rows_keys += max(0, L - ql + i + 1) if w.causal else L
    return 2.0 * w.num_heads * rows_keys * (576 + 512)


def timed_loop(fn, args, torch, stream):
    """Warm-up, then args.steps calls bracketed by events on `stream`: mean us."""
    warmup(fn, args.warmup, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / args.steps * 1e3


def time_schedule(w, ds, calls, schedule, args, torch, m, stream):
    """One schedule of one workload: the fused step, then each launch alone,
    with the dominant (stream) kernel's roofline."""
    kv_bytes = w.kv_bytes_touched()
    decs = [m.Decoder(**c, sinks=d["sinks"], schedule=schedule, out_dtype=torch.bfloat16)
            for c, d in zip(calls, ds)]
    us = timed_loop(lambda i: decs[i & 1].run(stream), args, torch, stream)
    stage_us = {st: timed_loop(lambda i, st=st: decs[i & 1].run_stage(st, stream), args, torch, stream)
                for st in (1, 2)}
    esz = 2 if w.kv_dtype == "bf16" else 1
    T, H = w.num_tokens, w.num_heads
    q_bytes = T * H * 576 * esz
    res = {"schedule": schedule, "us_per_step": round(us, 2),
           "eff_kv_GBps": round(kv_bytes / (us * 1e-6) / 1e9, 1),
           "kv_frac_of_hbm_peak": round(kv_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "stream_kernel_us": round(stage_us[1], 2), "merge_kernel_us": round(stage_us[2], 2)}
    if decs[0].split is not None:
        sched = split_schedule(w, *decs[0].split)
        alg = kv_bytes + q_bytes + sched["final_rows"] * (512 * 2 + 4) + sched["partial_rows"] * (512 * 2 + 8)
        kernel = "split_kernel"
        res["split"] = {"workgroups": decs[0].split[0], "rows_per_workgroup": decs[0].split[1],
                        "unit_keys": decs[0].split[2], **sched}
    else:
        S = decs[0].num_segments
        tile = w.tile_size or m.tile_size_for_block(w.block_size)
        qlen_r = [int(x) for x in (w.qo_indptr[1:] - w.qo_indptr[:-1])]
        valid = sum(ql * len(m.segment_bounds(int(L), S, tile)) for L, ql in zip(w.seq_lens, qlen_r))
        alg = kv_bytes + q_bytes + valid * H * (512 * 2 + 8)  # bf16 partials for the bf16 output
        kernel = "segment_kernel"
        res["num_segments"] = S
        res["segments_valid_rows"] = valid * H
    ach = alg / (stage_us[1] * 1e-6) / 1e9
    flops = attention_flops(w)
    peak_mfma = FP8_MFMA_PEAK_TFLOPS if w.kv_dtype != "bf16" else BF16_MFMA_PEAK_TFLOPS
    t_hbm = alg / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (peak_mfma * 1e12)
    if t_mfma > t_hbm:
        # more MFMA work than HBM traffic at the two peaks: the matrix cores bound it
        roof = {"bound": "mfma", "achieved": round(flops / (stage_us[1] * 1e-6) / 1e12, 1),
                "peak": peak_mfma, "unit": "TFLOP/s", "frac": round(t_mfma / (stage_us[1] * 1e-6), 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": profiled_traffic(w.name, schedule), "kernel": kernel,
                 "kernel_us": round(stage_us[1], 2), "algorithmic_bytes": int(alg),
                 "hbm_bytes_per_s": round(ach, 1), "flops": round(flops), "mfma_tflops": round(
                     flops / (stage_us[1] * 1e-6) / 1e12, 1)})
    res["roofline"] = roof
    del decs
    return res


def time_workload(name, args, torch, m, mi, schedules):
    """Every requested schedule of one workload on the same resident inputs."""
    w, ds = build_inputs(name, torch, mi)
    calls = [mi.call_args(w, d) for d in ds]
    stream = torch.cuda.current_stream()
    base = {"workload": name, "num_heads": w.num_heads, "dtype": w.kv_dtype,
            "num_reqs": w.num_reqs, "num_tokens": w.num_tokens, "max_qlen": w.max_qlen,
            "max_seq_len": w.max_seq_len, "block_size": w.block_size, "causal": bool(w.causal),
            "sinks": w.sinks is not None, "kv_bytes": w.kv_bytes_touched()}
    out = [dict(base, **time_schedule(w, ds, calls, sch, args, torch, m, stream)) for sch in schedules]
    del ds, calls
    torch.cuda.empty_cache()
    return w, out


def split_schedule(w, G, rows_wg, tt):
    """Rows the balanced split finishes in place and partial rows it writes,
    from the same unit layout the split kernel uses (request, row chunk, tile;
    workgroup g takes units [g W / G, (g+1) W / G))."""
    H = w.num_heads
    qo = [int(x) for x in w.qo_indptr]
    jobs = []  # (first unit, units, rows)
    off = 0
    for r, L in enumerate(int(x) for x in w.seq_lens):
        rows = (qo[r + 1] - qo[r]) * H
        nt = -(-L // tt) if L > 0 else 0
        nch = -(-rows // rows_wg) if nt else 0
        for c in range(nch):
            jobs.append((off + c * nt, nt, min(rows_wg, rows - c * rows_wg)))
        off += nch * nt
    W = off
    final_rows = partial_rows = pieces = 0
    for P, nt, rows in jobs:
        gf = ((P + 1) * G - 1) // W
        gl = ((P + nt) * G - 1) // W
        if gf == gl:
            final_rows += rows
        else:
            # workgroups with an empty range (G > W) hold no piece
            n = sum(1 for g in range(gf, gl + 1) if ((g + 1) * W) // G > (g * W) // G)
            pieces += n
            partial_rows += n * rows
    return {"units": W, "jobs": len(jobs), "final_rows": final_rows, "partial_rows": partial_rows,
            "split_pieces": pieces}


KERNEL_SOURCES = ("mla_paged_decode_02_amd/csrc/mla_kernels.hip", "mla_paged_decode_02_amd/csrc/mla_internal.h")


def profiled_traffic(workload, schedule="balanced"):
    """HBM bytes per stream-kernel launch from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary of this workload and schedule
    (copy-calibrated), or None when there is none or the kernel sources
    changed since it was taken."""
    import glob
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    digest = h.hexdigest()[:16]
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        kv = {}
        with open(path) as fh:
            for line in fh:
                if ":" in line and not line.startswith(("|", "#", " ")):
                    k, _, v = line.partition(":")
                    kv[k.strip()] = v.strip()
        if (kv.get("workload") == workload and kv.get("schedule", "balanced") == schedule
                and kv.get("kernel_source_sha256_16") == digest and "stream_kernel_traffic_bytes" in kv):
            return int(kv["stream_kernel_traffic_bytes"])
    return None


def cpu_baseline(w, nreq, min_runs=3, min_total_s=10.0, max_runs=15):
    """The fp64 oracle on the first `nreq` requests of the same batch (all of
    them by default), run at least `min_runs` times and until about
    `min_total_s` seconds of CPU work are done; the median run, scaled to GB/s
    of KV rows (the oracle as it stands, on the host cores)."""
    from oracle import mla_oracle as orc

    reqs = list(range(min(nreq, w.num_reqs) if nreq > 0 else w.num_reqs))
    times = []
    while len(times) < min_runs or (sum(times) < min_total_s and len(times) < max_runs):
        t = time.perf_counter()
        orc.mla_decode(w, reqs=reqs)
        times.append(time.perf_counter() - t)
    runs = len(times)
    dt = sorted(times)[len(times) // 2]
    esz = 2 if w.kv_dtype == "bf16" else 1
    rows = sum(int(w.seq_lens[r]) for r in reqs)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": round(rows * 576 * esz / dt / 1e9, 4), "unit": "GB/s (effective KV)", "cores": cores,
            "kind": "oracle",
            "sample": f"{len(reqs)} of {w.num_reqs} requests ({rows} KV rows, {w.num_heads} heads), fp64 NumPy "
                      f"oracle incl. page gather; median of {runs} runs: {dt:.2f} s per run "
                      f"({sum(times):.1f} s in all)"}


# The benchmark configurations of the decode measurements (bs=52 x 16K at
# 16..128 heads, and the ragged causal batch): each is timed under both
# schedules in the default run.
CORE = ["bs52_ctx16k_h16_bf16_blk64", "bs52_ctx16k_h16_fp8_blk64", "bs52_ctx16k_h48_fp8_blk64",
        "bs52_ctx16k_h64_fp8_blk64", "bs52_ctx16k_h128_bf16_blk256", "ragged128_max32k_h96_fp8_causal_sinks"]
OPTIONAL = ["bs52_ctx16k_h48_fp8_blk64_bf16q", "sparse_bs52_top2048_ctx16k_h16_bf16",
            "sparse_bs52_top2048_ctx16k_h128_fp8"]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (one GPU per box, "
              "no multi-GPU path in this library)", file=sys.stderr)
        sys.exit(2)
    import torch
    import mla_inputs as mi
    import mla_paged_decode_02_amd as m

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    m.lib()
    t0 = time.time()
    other = "segments" if args.schedule == "balanced" else "balanced"
    w, lines = time_workload(args.workload, args, torch, m, mi,
                             [args.schedule] if args.only else [args.schedule, other])
    head = lines[0]
    print(f"[bench] {args.workload} {args.schedule}: {head['us_per_step']} us/step", file=sys.stderr, flush=True)
    extra = lines[1:]
    if not args.only:
        names = [n for n in CORE if n != args.workload]
        if args.extra:
            names += [n for n in OPTIONAL if n != args.workload]
        for name in names:
            # both schedules for the benchmark configurations and the index
            # streams (where the planner's segments beat the balanced split)
            scheds = ["balanced", "segments"] if name in CORE or name.startswith("sparse") else ["balanced"]
            _, ls = time_workload(name, args, torch, m, mi, scheds)
            for ln in ls:
                print(f"[bench] {name} {ln['schedule']}: {ln['us_per_step']} us/step", file=sys.stderr,
                      flush=True)
            extra += ls
        if args.extra:
            for name in DCP_WORKLOADS:
                torch.cuda.empty_cache()
                extra.append(time_dcp(name, args, torch, m, mi))
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_sample_reqs)
    roof = dict(head["roofline"])
    line = {
        "metric": METRIC,
        "value": head["eff_kv_GBps"],
        "unit": "GB/s (effective KV bytes / step time)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_step"] / 1e3, 5),
        "us_per_step": head["us_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "fp8_e4m3",
        "data": "synthetic (seeded N(0,1) q and latent cache, random page permutation)",
        "config": {"workload": head["workload"], "schedule": head["schedule"], "batch": head["num_reqs"],
                   "tokens": head["num_tokens"], "max_qlen": head["max_qlen"],
                   "max_kv_tokens_per_request": head["max_seq_len"], "num_heads": head["num_heads"],
                   "block_size": head["block_size"], "causal": head["causal"], "sinks": head["sinks"],
                   "parallelism": "single GPU"},
        "kv_frac_of_hbm_peak": head["kv_frac_of_hbm_peak"],
        "roofline": roof,
        "stream_kernel_us": head["stream_kernel_us"],
        "merge_kernel_us": head["merge_kernel_us"],
        "split": head.get("split"),
        "cpu_baseline": cpu,
        "extra": extra,
        "wall_s": round(time.time() - t0, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
