#!/usr/bin/env python3
"""MLA paged decode benchmark on one MI355X.

One step = one full decode of the batch: the segment kernel (paged KV stream,
QK^T, base-2 online softmax, P.V, per-segment partials) and the merge kernel
(output + natural-log LSE), i.e. mla_decode through the C ABI.

Default workload: bs=52 requests, qlen=1, 16 heads, 16384 KV tokens per
request, bf16 q and latent cache ~N(0,1), block 64 = TILE 64, random block
table permutation, segment count from the planner, scale 1/sqrt(192).
Inputs are synthetic (seeded) and resident in HBM before timing starts; two
cache copies alternate between steps so no step reuses the previous step's
cache lines from the 256 MB last-level cache.

Prints ONE JSON line.  Extra configurations (--extra) are appended under
"extra" in the same line.
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
    ap.add_argument("--extra", action="store_true", help="also time the other bs=52 workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-reqs", type=int, default=0, help="requests the oracle times (0 = all)")
    ap.add_argument("--num-segments", type=int, default=0)
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
    decs = [m.Decoder(**mi.call_args(sw, d), sinks=None, num_segments=0, out=so[k], lse=sl[k])
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


def time_workload(name, args, torch, m, mi, want_roofline):
    w, ds = build_inputs(name, torch, mi)
    esz = 2 if w.kv_dtype == "bf16" else 1
    kv_bytes = w.kv_bytes_touched()
    calls = [mi.call_args(w, d) for d in ds]
    # One prepared call per cache copy: each step is a single C call.
    decs = [m.Decoder(**c, sinks=d["sinks"], num_segments=args.num_segments, out_dtype=torch.bfloat16)
            for c, d in zip(calls, ds)]
    S = decs[0].num_segments
    stream = torch.cuda.current_stream()

    def step(i):
        decs[i & 1].run(stream)

    warm_s = warmup(step, args.warmup, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    res = {"workload": name, "num_heads": w.num_heads, "dtype": w.kv_dtype, "num_segments": S,
           "split_workgroups": decs[0].split_workgroups,
           "num_reqs": w.num_reqs, "num_tokens": w.num_tokens, "max_qlen": w.max_qlen,
           "max_seq_len": w.max_seq_len, "block_size": w.block_size, "causal": bool(w.causal),
           "sinks": w.sinks is not None,
           "us_per_step": ms * 1e3, "kv_bytes": kv_bytes, "warmup_s": round(warm_s, 3),
           "eff_kv_GBps": kv_bytes / (ms * 1e-3) / 1e9,
           "frac_of_hbm_peak": kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if not want_roofline:
        return w, res, None

    T, H = w.num_tokens, w.num_heads
    out_esz = 2  # bf16 output
    q_bytes = T * H * 576 * esz
    if decs[0].split is not None:
        # Balanced split: stage 1 (the cache stream, the dominant kernel) and
        # stage 2 (the merge of requests cut by a range boundary), each timed
        # alone with events on the stream it is launched on.
        stage_us = {}
        for stage in (1, 2):
            warmup(lambda i: decs[i & 1].run_stage(stage, stream), args.warmup, torch)
            e0.record(stream)
            for i in range(args.steps):
                decs[i & 1].run_stage(stage, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            stage_us[stage] = e0.elapsed_time(e1) / args.steps * 1e3
        sched = split_schedule(w, *decs[0].split)
        alg = kv_bytes + q_bytes + sched["final_rows"] * (512 * out_esz + 4) + sched["partial_rows"] * (512 + 2) * 4
        kernel, kernel_us = "split_kernel", stage_us[1]
        res["split"] = {"workgroups": decs[0].split[0], "rows_per_workgroup": decs[0].split[1],
                        "unit_keys": decs[0].split[2], **sched}
        res["merge_kernel_us"] = stage_us[2]
    else:
        # Segment partition: segment kernel and merge kernel each timed alone.
        S = decs[0].num_segments
        so = torch.empty((T, H, S, 512), dtype=torch.float32, device="cuda")
        sm = torch.empty((T, H, S), dtype=torch.float32, device="cuda")
        se = torch.empty((T, H, S), dtype=torch.float32, device="cuda")
        warmup(lambda i: m.decode_segments(**calls[i & 1], num_segments=S, segm_output=so, segm_max=sm,
                                           segm_expsum=se, stream=stream), args.warmup, torch)
        e0.record(stream)
        for i in range(args.steps):
            m.decode_segments(**calls[i & 1], num_segments=S, segm_output=so, segm_max=sm,
                              segm_expsum=se, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        seg_ms = e0.elapsed_time(e1) / args.steps
        qlens = torch.diff(ds[0]["qo_indptr"])
        part_lens = torch.repeat_interleave(ds[0]["seq_lens"], qlens).to(torch.int32)
        mo = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
        ml = torch.empty((T, H), dtype=torch.float32, device="cuda")
        tile = w.tile_size or m.tile_size_for_block(w.block_size)
        warmup(lambda i: m.merge_segments(so, sm, se, part_lens, tile, sinks=ds[0]["sinks"], out=mo, lse=ml,
                                          stream=stream), args.warmup, torch)
        e0.record(stream)
        for i in range(args.steps):
            m.merge_segments(so, sm, se, part_lens, tile, sinks=ds[0]["sinks"], out=mo, lse=ml, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        res["merge_kernel_us"] = e0.elapsed_time(e1) / args.steps * 1e3
        qlen_r = [int(x) for x in (w.qo_indptr[1:] - w.qo_indptr[:-1])]
        valid = sum(ql * len(m.segment_bounds(int(L), S, tile)) for L, ql in zip(w.seq_lens, qlen_r))
        alg = kv_bytes + q_bytes + valid * H * (512 + 2) * 4
        kernel, kernel_us = "segment_kernel", seg_ms * 1e3
    achieved = alg / (kernel_us * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(name),
            "kernel": kernel, "kernel_us": round(kernel_us, 2), "algorithmic_bytes": int(alg)}
    res["segment_kernel_us"] = kernel_us
    return w, res, roof


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


def profiled_traffic(workload):
    """HBM bytes per segment-kernel launch from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary of this workload (copy-calibrated), or
    None when there is none or the kernel sources changed since it was taken."""
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
        if (kv.get("workload") == workload and kv.get("kernel_source_sha256_16") == digest
                and "stream_kernel_traffic_bytes" in kv):
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
    w, res, roof = time_workload(args.workload, args, torch, m, mi, want_roofline=True)
    extra = []
    if args.extra:
        for name in WORKLOADS:
            if name == args.workload:
                continue
            torch.cuda.empty_cache()
            _, r2, _ = time_workload(name, args, torch, m, mi, want_roofline=False)
            extra.append(r2)
        for name in DCP_WORKLOADS:
            torch.cuda.empty_cache()
            extra.append(time_dcp(name, args, torch, m, mi))
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_sample_reqs)
    line = {
        "metric": METRIC,
        "value": round(res["eff_kv_GBps"], 1),
        "unit": "GB/s (effective KV bytes / step time)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_s": res["warmup_s"],
        "ms_per_step": round(res["us_per_step"] / 1e3, 5),
        "us_per_step": round(res["us_per_step"], 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "fp8_e4m3",
        "data": "synthetic (seeded N(0,1) q and latent cache, random page permutation)",
        "config": {"workload": res["workload"], "batch": res["num_reqs"], "tokens": res["num_tokens"],
                   "max_qlen": res["max_qlen"], "max_kv_tokens_per_request": res["max_seq_len"],
                   "num_heads": res["num_heads"], "block_size": res["block_size"],
                   "causal": res["causal"], "sinks": res["sinks"],
                   "num_segments": res["num_segments"], "split_workgroups": res["split_workgroups"],
                   "parallelism": "single GPU"},
        "frac_of_hbm_peak": round(res["frac_of_hbm_peak"], 4),
        "roofline": roof,
        "stream_kernel_us": round(res.get("segment_kernel_us", 0.0), 2),
        "merge_kernel_us": round(res.get("merge_kernel_us", 0.0), 2),
        "split": res.get("split"),
        "cpu_baseline": cpu,
        "extra": extra,
        "wall_s": round(time.time() - t0, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
