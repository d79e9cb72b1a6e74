#!/usr/bin/env python3
"""Benchmark of the JointSchemaHead forward pass on one MI355X.

One step = one clef_head_forward over one batch of the online-serving
workload (B=8 records padded to L=4096, valid lengths U{2048..4096}, H=4096,
8 fields per record, full 248320-row lexical table), with hidden states and
the table already resident in HBM.  As a serving loop would, the timed steps
keep --in-flight batches in flight (default 2): that many heads share one set
of device weights (clef_head_create_sharing), each with its own inputs,
workspace and stream, and step i runs on head i mod n, so one batch's
latency-bound small-GEMM chain overlaps the next batch's big GEMMs.  The
same K steps on a single head and stream are timed too (one batch at a
time: the per-batch latency), with HIP events around every forward on its
stream for the median and p95 latency, once warm (back-to-back) and once
cold (a 512 MiB buffer written between forwards, so the ~210 MB of weights
no longer sit in the 256 MB memory-side cache).  Prints one JSON line:
records/s for the whole job, latency statistics, per-stage GPU times from
HIP events recorded on the forward's stream with each stage's fraction of
its roofline, the roofline of the dominant kernel, and the fp64 oracle timed
on the host cores over a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--config 1] [--in-flight 2] [--precision bf16|f32]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
COLD_BYTES = 512 << 20         # written between forwards for the cold-cache latency

WORKLOADS = {
    0: "single record: B=1, L=160, H=4096, 1 noul + 1 choice field, V=8192",
    1: "online-serving batch: B=8, L=4096 padded, valid U{2048..4096}, H=4096, 8 fields/record "
       "(3 noul, 3 choice of 2-6, 2 score of 5), V=248320",
    2: "long state: B=1, L=16384, H=4096, 4 fields (15 options), V=248320",
    3: "wide schema: B=4, L=8192, H=4096, 32 fields/record (8 noul, 16 choice of 4-16, 8 score), V=248320",
    4: "heterogeneous large backbone: B=32, H=5120, valid log-uniform [512, 16384], 1-16 fields, V=248320",
}
WORKLOAD_SLUGS = {0: "single_record_l160", 1: "online_serving_b8_l4096", 2: "long_state_l16384",
                  3: "wide_schema_b4_l8192", 4: "heterogeneous_b32_h5120"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sources_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "structured_decision_head_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(stage, cfg_index):
    """HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE, WRITE_SIZE),
    scaled by the copy-kernel calibration; None if absent or stale."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{WORKLOAD_SLUGS[cfg_index]}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != kernel_sources_sha(t.get("sources", [])):
        return None
    return t.get("bytes_per_launch")


def host_info():
    """Core count, affinity, CPU model and BLAS library of the host the oracle runs on."""
    from threadpoolctl import threadpool_info
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
            for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"host_cpu_count": os.cpu_count(), "host_affinity_cores": len(os.sched_getaffinity(0)),
            "cpu_model": model, "blas": ", ".join(blas) or None}, threads


def latency(runner, stream, k, torch, np, cold=None):
    """Median and p95 (us) of k forwards one at a time on one stream, each
    bracketed by HIP events on that stream; with `cold`, the buffer is written
    on the same stream before every forward (outside the bracket)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k)]
    with torch.cuda.stream(stream):
        for i in range(k):
            if cold is not None:
                cold.fill_(i & 0xff)
            ev[i][0].record(stream)
            runner.forward(stream)
            ev[i][1].record(stream)
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
    return {"median": round(float(np.median(d)), 1), "p95": round(float(np.percentile(d, 95)), 1), "steps": k}


def streamed_ingest(args, C, HeadRunner, case, runner, torch, np, H):
    """The same batch fed as the backbone's chunked prefill emits it (varlen, 64-row
    chunks, chunk k of every record before chunk k + 1); returns the median time the
    head needs after the last chunk (clef_head_stream_end) and for the whole stream."""
    b = case.batch
    sr = HeadRunner(case, share=runner)
    sr.set_batch(None, C.CLEF_VARLEN)
    sst = torch.cuda.Stream()
    cu = b.cu_seqlens()
    chunks = []
    pos = [0] * b.B
    while any(pos[k] < b.lengths[k] for k in range(b.B)):
        for k in range(b.B):
            if pos[k] < b.lengths[k]:
                n = int(min(64, b.lengths[k] - pos[k]))
                chunks.append((k, pos[k], n, sr.hidden.data_ptr() + (int(cu[k]) + pos[k]) * H * 2))
                pos[k] += n
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tails, totals = [], []
    for it in range(args.warmup + max(args.steps // 5, 5)):
        ev[0].record(sst)
        C.clef_head_stream_begin(sr.handle, sr.args, sst.cuda_stream)
        for k, p0, n, ptr in chunks:
            C.clef_head_stream_rows(sr.handle, k, p0, n, ptr, sst.cuda_stream)
        ev[1].record(sst)
        C.clef_head_stream_end(sr.handle, sr.args, sr.logits.data_ptr(), sr.probs.data_ptr(), sr.argmax.data_ptr(),
                               sst.cuda_stream)
        ev[2].record(sst)
        ev[2].synchronize()
        if it >= args.warmup:
            tails.append(ev[1].elapsed_time(ev[2]))
            totals.append(ev[0].elapsed_time(ev[2]))
    sr.close()
    return {"chunk_rows": 64, "chunks": len(chunks), "tail_us": round(float(np.median(tails)) * 1e3, 1),
            "total_us": round(float(np.median(totals)) * 1e3, 1)}


def library_gemm(args, torch, synth):
    """torch.matmul (hipBLASLt) on the two big products of the workload, over the
    same 256-row tile space the head's GEMMs cover; W given as the transposed
    view of [out, in] rows (the faster of the two operand forms measured)."""
    case = synth.config_case(args.config, with_table=False)
    b = case.batch
    rows = 256 * sum(-(-int(n) // 256) for n in b.lengths)
    H, D = case.head.hidden_size, case.head.width
    out = {"library_gemm": "torch.matmul bf16 (hipBLASLt), median of 20", "config": args.config, "rows": rows}
    torch.manual_seed(0)
    for name, M, N, K in (("memory", rows, D, H), ("kv", rows, 2 * D * case.head.routing_layers, D)):
        a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        w = torch.randn(N, K, device="cuda", dtype=torch.bfloat16)
        for _ in range(5):
            c = torch.matmul(a, w.t())
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(20):
            s.record()
            c = torch.matmul(a, w.t())
            e.record()
            torch.cuda.synchronize()
            ts.append(s.elapsed_time(e) * 1e3)
        us = sorted(ts)[len(ts) // 2]
        out[name] = {"M": M, "N": N, "K": K, "us": round(us, 1), "tflops": round(2.0 * M * N * K / us / 1e6, 1)}
        del a, w, c
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--in-flight", type=int, default=2, help="batches in flight (heads sharing weights)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--field-cross-attention", action="store_true",
                    help="decoder-layer reading of the field layers (cross-attention over the memory rows)")
    ap.add_argument("--hidden", choices=("bf16", "f16"), default="bf16",
                    help="element type of the hidden states (f16: the CoreML packaging's fp16 hidden)")
    ap.add_argument("--precision", choices=("bf16", "f32"), default="bf16",
                    help="arithmetic of the head (f32: CLEF_PRECISION_F32)")
    ap.add_argument("--cold-steps", type=int, default=30, help="forwards of the cold-cache latency (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream", action="store_true", help="skip the streamed-ingest measurement")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (HBM counter calibration)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time the vendor GEMM (torch.matmul, hipBLASLt) on the shapes of the workload's "
                         "memory and K/V products, plain bf16 with no epilogue: a comparison point")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only (the head shards by record with no exchange between GPUs: "
              "N GPUs run N independent heads); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from structured_decision_head_amd import clefhead as C
    from structured_decision_head_amd import synth
    from structured_decision_head_amd.runner import HeadRunner

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 5}), flush=True)
        return
    if args.library_gemm:
        library_gemm(args, torch, synth)
        return
    t = time.time()
    f32 = args.precision == "f32"
    case = synth.config_case(args.config, hidden_dtype=args.hidden,
                             field_cross_attention=int(args.field_cross_attention), precision=int(f32))
    b = case.batch
    H, D = case.head.hidden_size, case.head.width
    T = int(b.lengths.sum())
    log(f"generated workload {args.config} in {time.time() - t:.1f}s: B={b.B} L={b.L} T={T} NQ={b.NQ} NO={b.NO}")

    if args.in_flight < 1:
        log("--in-flight must be >= 1")
        sys.exit(2)
    runner = HeadRunner(case)
    runner.set_batch()
    h = runner.handle
    runners = [runner]
    for _ in range(args.in_flight - 1):
        r = HeadRunner(case, share=runner)
        r.set_batch()
        runners.append(r)
    streams = [torch.cuda.Stream() for _ in runners]

    def steps(n, k):
        for i in range(k):
            runners[i % n].forward(streams[i % n])

    def timed(n):
        steps(n, args.warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        steps(n, args.steps)     # host validation and table upload included
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    # timed region: K forwards with in_flight batches in flight, then the same K one at a time
    ms_per_step = timed(len(runners))
    ms_one = timed(1) if len(runners) > 1 else ms_per_step
    log(f"{ms_per_step * 1e3:.1f} us per forward with {len(runners)} in flight; {ms_one * 1e3:.1f} us one at a time")
    # latency per forward (HIP events), warm and cold
    lat = latency(runner, streams[0], args.steps, torch, np)
    cold = None
    if args.cold_steps > 0:
        buf = torch.empty(COLD_BYTES, dtype=torch.uint8, device="cuda")
        cold = latency(runner, streams[0], args.cold_steps, torch, np, cold=buf)
        cold["between_forwards"] = "512 MiB written by a fill kernel on the forward's stream"
        del buf
    log(f"latency us: warm {lat}, cold {cold}")

    # per-stage GPU time over the same number of forwards (events on the forward's stream)
    C.clef_head_set_profiling(h, True)
    for _ in range(args.steps):
        runner.forward()
    stage_ms, nfw = C.clef_head_stage_times(h)
    C.clef_head_set_profiling(h, False)
    stage_us = {k: v * 1e3 / nfw for k, v in stage_ms.items()}

    # streamed ingest of the same batch (varlen, 64-row chunks as the backbone's chunked prefill
    # emits them, chunk k of every record before chunk k + 1): the work left after the last chunk
    # (clef_head_stream_end) is the head's latency once the backbone is done
    stream = None
    if not args.no_stream and not f32:   # streamed ingest runs in the bf16 mode only
        stream = streamed_ingest(args, C, HeadRunner, case, runner, torch, np, H)
        log(f"streamed ingest: {stream}")
    log("stage us: " + ", ".join(f"{k}={v:.1f}" for k, v in stage_us.items()))
    lg, pr, am = runner.outputs()

    NR, NL = case.head.routing_layers, case.head.layers
    # the K/V stage also computes the field layers' cross K/V in the decoder-layer variant
    kv_layers = NR + (NL if args.field_cross_attention else 0)
    gemm_flops = {"memory_gemm": 2.0 * T * H * D, "kv_gemm": 2.0 * T * D * (2 * D * kv_layers)}
    dominant = max(gemm_flops, key=lambda k: stage_us[k])
    achieved = gemm_flops[dominant] / (stage_us[dominant] * 1e-6) / 1e12
    # counters were taken on the bf16 big-GEMM kernels; the fp16 memory GEMM and the fp32 mode's are others
    traffic = (load_traffic(dominant, args.config)
               if not f32 and (args.hidden == "bf16" or dominant != "memory_gemm") else None)
    # fp32 mode: every fp32 product runs as three bf16 MFMA terms, so its ceiling is a third of the bf16 rate
    peak = PEAK_BF16_TFLOPS / 3.0 if f32 else PEAK_BF16_TFLOPS
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(achieved, 1), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic}
    if traffic is not None:
        roofline["traffic_basis"] = ("FETCH_SIZE + WRITE_SIZE per launch, copy-calibrated: L2-to-fabric bytes, "
                                     "memory-side (MALL) cache hits included")
    if f32:
        roofline["peak_basis"] = (f"bf16 MFMA {PEAK_BF16_TFLOPS} TFLOP/s / 3 bf16 terms per fp32 product "
                                  f"(fp32 MFMA peak: {PEAK_F32_MFMA_TFLOPS})")
    stages = {k: {"us": round(v, 2)} for k, v in stage_us.items()}
    for k, fl in gemm_flops.items():
        stages[k]["tflops"] = round(fl / (stage_us[k] * 1e-6) / 1e12, 1)
        stages[k]["frac_mfma"] = round(fl / (stage_us[k] * 1e-6) / 1e12 / peak, 4)
    # algorithmic bytes of the HBM-bound stages: hidden rows once (row statistics), span rows and
    # global rows (pooling), lexical-table rows (gather), K and V of every layer (routing attention)
    span_rows = int((b.q_span[:, 1] - b.q_span[:, 0]).sum() + (b.o_span[:, 1] - b.o_span[:, 0]).sum()) + b.B
    kv_el = 4 if f32 else 2
    hbm = {"rowstats": 2.0 * T * H, "pool": 2.0 * span_rows * H, "lexical": 2.0 * H * len(b.o_ids),
           "route_attn": kv_el * 2.0 * T * D * NR}
    for k, by in hbm.items():
        gbs = by / (stage_us[k] * 1e-6) / 1e9
        stages[k]["gbs"] = round(gbs, 1)
        stages[k]["frac_hbm"] = round(gbs / PEAK_HBM_GBS, 4)

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import head as O
        params = O.load_params(case.weights)
        # cycle through the batch's records until the time budget is spent
        done, outs, t0 = [], [], time.perf_counter()
        while True:
            r = len(done) % b.B
            outs.append(O.forward(case.weights, case.head, b, lambda ids: case.table[np.asarray(ids, np.int64)],
                                  records=[r], params=params))
            done.append(r)
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        el = time.perf_counter() - t0
        hinfo, threads = host_info()
        # the first pass over the records also checks the GPU outputs
        first = done[:b.B]
        o0 = [int(b.o_offsets[b.q_offsets[r]]) for r in first]
        o1 = [int(b.o_offsets[b.q_offsets[r + 1]]) for r in first]
        gl = np.concatenate([lg[a:c] for a, c in zip(o0, o1)])
        gp = np.concatenate([pr[a:c] for a, c in zip(o0, o1)])
        ol = np.concatenate([o[0] for o in outs[:len(first)]])
        op = np.concatenate([o[1] for o in outs[:len(first)]])
        cpu = {"value": round(len(done) / el, 3), "unit": "records/s", "cores": threads, "kind": "oracle",
               "sample": f"{len(done)} record forwards cycling over the batch's {b.B} records, fp64 NumPy, {el:.1f}s",
               "max_abs_dlogit_vs_gpu": float(np.abs(gl - ol).max()),
               "max_abs_dprob_vs_gpu": float(np.abs(gp - op).max()), **hinfo}
        log(f"oracle: {cpu}")

    for r in runners[::-1]:
        r.close()
    value = b.B / (ms_per_step * 1e-3)
    line = {
        "metric": "records/s (JointSchemaHead forward; also us/record)",
        "value": round(value, 1),
        "unit": "records/s",
        "us_per_record": round(ms_per_step * 1e3 / b.B, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "in_flight": len(runners),
        "ms_per_batch_one_in_flight": round(ms_one, 4),
        "records_per_s_one_in_flight": round(b.B / (ms_one * 1e-3), 1),
        "latency_us": {**lat, "timer": "HIP events around each forward on its stream, one batch at a time"},
        "latency_cold_us": cold,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("f32" + ("" if args.hidden == "bf16" else " (fp16 hidden)")) if f32 else
                 ("bf16" if args.hidden == "bf16" else "f16 hidden, bf16 weights"),
        "data": "synthetic (seeded; random-init head weights, N(0,1) hidden states, N(0,0.02) lexical table)",
        "config": {"workload": WORKLOADS[args.config] + ("" if args.hidden == "bf16" else ", fp16 hidden states")
                   + (", decoder-layer fields" if args.field_cross_attention else "")
                   + (", fp32 head (CLEF_PRECISION_F32)" if f32 else ""),
                   "global_batch": int(b.B),
                   "seq_len": int(b.L), "valid_rows": T, "questions": int(b.NQ), "options": int(b.NO)},
        "roofline": roofline,
        "streamed_ingest": stream,
        "stages": stages,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
