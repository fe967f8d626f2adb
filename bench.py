"""Benchmark: append + decode attention over a quantized KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--layers L] [--no-cpu-baseline] [--no-others]
    python bench.py --summarize-profiles DIR      (rebuild profiles/*.md)

The default workload is ``verify``: 2 sessions of 131072 cached rows, 16 Q /
4 KV heads of 256 dims, 8 causal query rows per step, then the rollback to
len + 3 -- the long-context shape the bandwidth target is quoted at.

A step is one pass of the whole hot path over one layer cache: the fused
quantize-and-append of T rows per session, the split-K decode plus the
log-sum-exp combine of the T query rows, and the step's length bookkeeping
(truncate back to the steady length, or the verify rollback).  Steps rotate
over L independent layer caches so that the KV footprint exceeds the 256 MB
MALL and the reads come from HBM.  Inputs are seeded synthetic tensors,
resident on the GPU before timing starts.

Prints ONE JSON line.  ``value`` is the effective KV read bandwidth of the
whole step (algorithmic K+V bytes the decode must read / wall time per step,
steps replayed as captured HIP graphs).  ``roofline`` is that of the
dominant kernel, the split-K decode (partials) kernel: algorithmic K+V bytes
per launch / its mean duration, timed live with HIP events that the library
records on its own stream right before and after the kernel
(kvq_set_trace_events), against the 8 TB/s HBM peak; it also carries the
whole decode call (partials + combine, timed as back-to-back batches with no
host work between calls) and both fractions against a streaming-read ceiling
measured in the same run (libkvq_probe, a plain read of >= 2 GiB).
``traffic`` is the HBM bytes per decode call from the committed rocprofv3
FETCH_SIZE / WRITE_SIZE passes (profiles/decode_traffic.json), reported only
while the kernel sources still hash to the measured state.  ``cpu_baseline``
times the CPU oracle (one thread and all threads) on a bounded sample of the
same workload.  ``other_workloads`` repeats the GPU measurement for every
other workload, each with its own roofline object.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "decode attn effective KV GB/s (% of HBM peak) + steps/s; append tokens/s"
MALL_BYTES = 256 << 20
DTYPE = "fp16 MFMA operands (bf16/fp32 inputs, q8_0/q5_1 codes), fp32 accumulation and softmax"
PROBE_BYTES = 4 << 30


def source_hash() -> str:
    """sha256 (first 16 hex) over the library's kernel and host sources, in
    name order (the measurement probe excluded)."""
    import hashlib
    d = os.path.join(ROOT, "decode_attention_quantized_append_amd", "csrc")
    h = hashlib.sha256()
    for n in sorted(os.listdir(d)):
        if n.endswith((".hip", ".cpp", ".h")) and n != "kvq_probe.hip":
            h.update(n.encode())
            with open(os.path.join(d, n), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per decode call (partials + combine kernels) from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE passes, scaled by the copy
    calibration; None when the sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash() or workload not in t.get("workloads", {}):
        return None
    return round(t["workloads"][workload]["call_bytes"])


def default_layers(w) -> int:
    per_layer = w.kv_bytes_per_decode()
    if per_layer < (1 << 20):
        return 1                              # launch-bound; no footprint can matter
    return max(2, min(256, math.ceil(4 * MALL_BYTES / per_layer)))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="verify")
    ap.add_argument("--layers", type=int, default=0)
    ap.add_argument("--split-rows", type=int, default=0)
    ap.add_argument("--tiling", default="", metavar="KERNEL,HEAD_GROUP[,SUB]",
                    help="decode kernel (1 per-head, 3 stream), KV heads per "
                         "workgroup and sub_tiles, as kvq_set_decode_tiling; default: the "
                         "library's choice")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other workloads (each timed after the main one, with "
                         "--other-steps steps)")
    ap.add_argument("--other-steps", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--graph", choices=("auto", "on", "off"), default="auto",
                    help="replay each step as one captured HIP graph (auto and on: every "
                         "workload; verify rounds, whose lengths grow, in graph mode)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES, 10 times "
                         "(reference for scaling HBM traffic counters)")
    ap.add_argument("--summarize-profiles", default="", metavar="DIR",
                    help="only write profiles/*.md from the rocprofv3 outputs under DIR "
                         "(the layout the commands in those files produce)")
    return ap.parse_args()


def calibrate_copy(nbytes: int):
    import torch
    dev = torch.device("cuda:0")
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    dt = (time.perf_counter() - t0) / 10
    print(json.dumps({"calibrate_copy_bytes": nbytes, "read_bytes": nbytes, "write_bytes": nbytes,
                      "ms": round(dt * 1e3, 4), "GBps_read_plus_write": round(2 * nbytes / dt / 1e9, 1)}))


def stream_read_ceiling(nbytes: int = PROBE_BYTES):
    """The read bandwidth a plain streaming kernel sustains over nbytes of
    HBM (libkvq_probe): the best of a few launch shapes, each timed over 5
    passes with HIP events."""
    import torch

    from decode_attention_quantized_append_amd import build as kb
    lib = ctypes.CDLL(kb.LIB_PROBE)
    lib.kvq_probe_stream_read.restype = ctypes.c_int
    lib.kvq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(3)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(cus * 32 * 4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    best = None
    for per_cu in (4, 8, 16, 32):
        for unroll in (4, 8):
            blocks = cus * per_cu
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            rc = lib.kvq_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, unroll, stream)
            assert rc == 0, "probe launch failed"
            e0.record()
            for _ in range(5):
                lib.kvq_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, unroll, stream)
            e1.record()
            torch.cuda.synchronize(dev)
            gbps = 5 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if best is None or gbps > best["GBps"]:
                best = {"GBps": round(gbps, 1), "bytes": nbytes, "workgroups": blocks, "loads_in_flight": unroll}
    del buf
    torch.cuda.empty_cache()
    return best


def build_layers(w, L, dev, split_rows, tiling="", grow_rows=8 * 1024, graph_mode=False):
    import torch

    from decode_attention_quantized_append_amd import KvqLayerCache
    cap = w.capacity(extra_steps=0) if w.ring_cap else int(w.lengths().max()) + grow_rows
    caches = [KvqLayerCache(w.B, w.H, w.Hkv, w.hd, cap, w.window, w.ring_step, device=dev, fmt=w.fmt)
              for _ in range(L)]
    if graph_mode:
        # decode plans for every length the plane allows, so that one
        # captured round replays while the lengths grow
        for c in caches:
            c.set_graph_mode(True)
    tdt = torch.bfloat16 if w.io_dtype == "bf16" else torch.float32
    for counts, starts, T in w.prefill_pieces():
        k, v = w.kv_block(counts, starts, T)
        kd = torch.from_numpy(k).to(tdt).to(dev)
        vd = torch.from_numpy(v).to(tdt).to(dev)
        for c in caches:
            c.append(kd, vd, counts.tolist())
    for c in caches:
        if split_rows:
            c.set_split_rows(split_rows)
        if tiling:
            parts = [int(x) for x in tiling.split(",")]
            c.set_decode_tiling(parts[0], parts[1], parts[2] if len(parts) > 2 else 0)
    torch.cuda.synchronize(dev)
    return caches, cap


def _events(n):
    """n timing events, each recorded once so that the HIP event exists."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record()
    return ev


def run_gpu(w, args):
    import torch
    dev = torch.device("cuda:0")
    L = args.layers or default_layers(w)
    # verify rounds keep rollback_keep rows each: the planes are sized to the
    # rows this run adds (eager and replayed rounds), so that graph-mode plans
    # cover little more than the real lengths
    growing = bool(w.rollback_keep)
    rounds = -(-3 * (args.warmup + args.steps) // L) + 10
    grow = w.rollback_keep * rounds + w.T + 64 if growing else 8 * 1024
    caches, cap = build_layers(w, L, dev, args.split_rows, args.tiling, grow_rows=grow,
                               graph_mode=growing and args.graph != "off")
    tdt = torch.bfloat16 if w.io_dtype == "bf16" else torch.float32
    pre = w.pre_step_lengths()
    k, v = w.kv_block([w.T] * w.B, pre, w.T)
    k_step = torch.from_numpy(k).to(tdt).to(dev)
    v_step = torch.from_numpy(v).to(tdt).to(dev)
    q = torch.from_numpy(w.q(0)).to(tdt).to(dev)
    s = w.sink_logits()
    sinks = torch.from_numpy(s).to(dev) if s is not None else None
    B, T, H, hd = w.B, w.T, w.H, w.hd
    out = torch.empty((B, T, H, hd), dtype=torch.float32, device=dev)
    lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    # workspace sized for the largest plan any step can need (lengths grow in
    # the ring and verify workloads; plans depend only on lengths)
    ws_bytes = 0
    for c in caches:
        ws_bytes = max(ws_bytes, 4 * c.workspace(T).numel())

    # Pre-bound C calls: the timed loops do no Python work beyond the calls.
    lib = caches[0].lib
    stream = torch.cuda.current_stream(dev).cuda_stream or None
    dt = caches[0]._dtype(q)
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)
    ws_ptr = ws.data_ptr() + (-ws.data_ptr()) % 256
    pre_arr = (ctypes.c_int32 * B)(*[int(x) for x in pre])
    sink_ptr = sinks.data_ptr() if sinks is not None else None
    kp, vp, qp, op, lp = k_step.data_ptr(), v_step.data_ptr(), q.data_ptr(), out.data_ptr(), lse.data_ptr()
    drop_arr = (ctypes.c_int32 * B)(*([w.T - w.rollback_keep] * B))
    scale = ctypes.c_float(w.scale)

    def check(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {lib.kvq_last_error().decode()}")

    def one_step(i, ev=None, st=None):
        st = stream if st is None else st
        h = caches[i % L].h
        if ev is not None:
            ev[0].record()
        check(lib.kvq_append(h, kp, vp, dt, T, None, st), "append")
        if ev is not None:
            ev[1].record()
        check(lib.kvq_decode(h, qp, dt, T, sink_ptr, scale, op, lp, ws_ptr, ws_bytes, st), "decode")
        if w.rollback_keep:                        # verify: keep rollback_keep of the T rows
            check(lib.kvq_rollback(h, drop_arr, st), "rollback")
        else:                                      # steady length: drop the step's rows (a ring
            check(lib.kvq_truncate(h, pre_arr, st), "truncate")   # keeps its window resident)

    # every layer takes at least one untimed step: a ring's first step after
    # the setup appends may rebase it (host-planned row moves), which the
    # timed steps of a steady state do not
    for i in range(max(args.warmup, L)):
        one_step(i)
    torch.cuda.synchronize(dev)

    # (1) per-kernel times: eager steps, the library recording events right
    # before its partials kernel, between it and the combine, and after it
    n_ev = args.steps
    ev_app = [_events(2) for _ in range(n_ev)]
    ev_dec = [_events(3) for _ in range(n_ev)]
    for i in range(n_ev):
        h = caches[(args.warmup + i) % L].h
        check(lib.kvq_set_trace_events(h, ev_dec[i][0].cuda_event, ev_dec[i][1].cuda_event,
                                       ev_dec[i][2].cuda_event), "trace events")
        one_step(args.warmup + i, ev_app[i])
    torch.cuda.synchronize(dev)
    for c in caches:
        check(lib.kvq_set_trace_events(c.h, None, None, None), "trace events")
    app_ms = [e[0].elapsed_time(e[1]) for e in ev_app]
    part_ms = [e[0].elapsed_time(e[1]) for e in ev_dec]
    comb_ms = [e[1].elapsed_time(e[2]) for e in ev_dec]

    # (2) the decode call (partials + combine) as back-to-back batches over
    # the layers, with no host work between the calls, on each layer's state
    # after a step's append (a ring's T query rows see rows that the
    # truncate to the pre-step length leaves behind base)
    for c in caches:
        check(lib.kvq_append(c.h, kp, vp, dt, T, None, stream), "append")
    reps = max(1, -(-args.steps // L))
    calls = reps * L
    e0, e1 = _events(2)
    e0.record()
    for i in range(calls):
        check(lib.kvq_decode(caches[i % L].h, qp, dt, T, sink_ptr, scale, op, lp, ws_ptr, ws_bytes, stream),
              "decode")
    e1.record()
    torch.cuda.synchronize(dev)
    call_ms = e0.elapsed_time(e1) / calls
    for c in caches:
        if w.rollback_keep:
            check(lib.kvq_rollback(c.h, drop_arr, stream), "rollback")
        else:
            check(lib.kvq_truncate(c.h, pre_arr, stream), "truncate")

    # (3) whole steps: one captured graph per layer, replayed
    use_graph = args.graph != "off"
    if use_graph:
        cap_st = torch.cuda.Stream(dev)
        steps_g = []
        for li in range(L):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap_st):
                one_step(li, st=cap_st.cuda_stream)
            steps_g.append(g)
        for i in range(args.warmup):
            steps_g[i % L].replay()
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for i in range(args.steps):
            steps_g[(args.warmup + i) % L].replay()
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - t0
    else:
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for i in range(args.steps):
            one_step(args.warmup + i)
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - t0
    if growing:   # replays moved the device lengths: bring the host mirrors back in step
        for c in caches:
            ln, bs, overflow = c.device_lengths()
            assert overflow == 0, "a replayed round did not fit its plane"
            c.set_host_lengths(ln, bs)

    # attention importance of a step's query rows (an optional extra pass:
    # it re-reads the K rows the step sees), timed with HIP events on a few
    # layers after a decode of the same rows supplied the log-sum-exps
    imp = torch.zeros((B, cap), dtype=torch.float32, device=dev)
    imp_ms = []
    for li in range(min(L, 8)):
        h = caches[li].h
        i0, i1 = _events(2)
        check(lib.kvq_append(h, kp, vp, dt, T, None, stream), "append")
        check(lib.kvq_decode(h, qp, dt, T, sink_ptr, scale, op, lp, ws_ptr, ws_bytes, stream), "decode")
        i0.record()
        check(lib.kvq_importance(h, qp, dt, T, scale, lp, imp.data_ptr(), stream), "importance")
        i1.record()
        if w.rollback_keep:
            check(lib.kvq_rollback(h, drop_arr, stream), "rollback")
        else:
            check(lib.kvq_truncate(h, pre_arr, stream), "truncate")
        torch.cuda.synchronize(dev)
        imp_ms.append(i0.elapsed_time(i1))
    rebase = None
    if w.ring_cap:
        # the ring's rebase, off the steady path: fill a layer's plane, then
        # time the append that has to move the live rows down first (HIP
        # events around the library call), against a plain append
        one = (ctypes.c_int32 * B)(*([1] * B))
        times = []
        for li in range(min(L, 16)):
            h = caches[li].h
            room = min(cap - (int(x) - int(y)) for x, y in zip(*caches[li].host_lengths()))
            for _ in range(room):
                check(lib.kvq_append(h, kp, vp, dt, T, one, stream), "append")
            r0, r1 = _events(2)
            base0 = caches[li].host_lengths()[1][0]
            r0.record()
            check(lib.kvq_append(h, kp, vp, dt, T, one, stream), "append with rebase")
            r1.record()
            torch.cuda.synchronize(dev)
            assert caches[li].host_lengths()[1][0] > base0, "the append did not rebase"
            times.append(r0.elapsed_time(r1))
        ln, bs = caches[0].host_lengths()
        rebase = dict(append_with_rebase_ms=round(sum(times) / len(times), 5),
                      rows_moved_per_session=int(ln[0] - 1 - bs[0]), ring_step=w.ring_step,
                      amortized_ms_per_append=round((sum(times) / len(times) - sum(app_ms) / len(app_ms))
                                                    / w.ring_step, 6))
    srt = sorted(part_ms)
    return dict(L=L, cap=cap, ms_step=wall * 1e3 / args.steps, graph=use_graph, rebase=rebase,
                app_ms=sum(app_ms) / len(app_ms), part_ms=sum(part_ms) / len(part_ms),
                part_p10=srt[len(srt) // 10], part_p90=srt[(9 * len(srt)) // 10],
                comb_ms=sum(comb_ms) / len(comb_ms), call_ms=call_ms, calls=calls,
                imp_ms=sum(imp_ms) / len(imp_ms), kv_bytes=w.kv_bytes_per_decode(), ws_bytes=ws_bytes,
                footprint=L * (caches[0].sizes.k_planes_bytes + caches[0].sizes.v_planes_bytes))


def importance_summary(w, r):
    """The importance pass reads the K rows of the step's span once."""
    kbytes = int(w.span().sum()) * w.k_row_bytes
    return {"ms": round(r["imp_ms"], 5), "k_bytes": kbytes,
            "GBps": round(kbytes / (r["imp_ms"] * 1e-3) / 1e9, 2)}


def roofline(w, r, ceiling):
    """Roofline of the dominant kernel (the split-K partials kernel) and of
    the whole decode call, from the live event times."""
    kv = r["kv_bytes"]
    ach = kv / (r["part_ms"] * 1e-3) / 1e9
    call = kv / (r["call_ms"] * 1e-3) / 1e9
    ro = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
          "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(w.name),
          "traffic_unit": "HBM bytes per decode call (partials + combine), rocprofv3 counters",
          "algorithmic": kv, "algorithmic_unit": "K+V bytes of the rows the step's query rows see",
          "kernel": "split-K decode partials kernel (kvq_decode's first launch)",
          "kernel_ms": {"mean": round(r["part_ms"], 5), "p10": round(r["part_p10"], 5),
                        "p90": round(r["part_p90"], 5)},
          "combine_ms": round(r["comb_ms"], 5),
          "call": {"ms": round(r["call_ms"], 5), "achieved": round(call, 2),
                   "frac": round(call / HBM_PEAK_GBPS, 4),
                   "timing": f"{r['calls']} back-to-back kvq_decode calls between two HIP events"}}
    if ceiling:
        ro["ceiling"] = {"GBps": ceiling["GBps"], "kernel_frac": round(ach / ceiling["GBps"], 4),
                         "call_frac": round(call / ceiling["GBps"], 4)}
    if w.T * w.hpk > 32:   # a prompt chunk: a real contraction, also reported against the fp16 MFMA peak
        tf = w.attn_flops_per_decode() / (r["part_ms"] * 1e-3) / 1e12
        ro["mfma"] = {"TFLOPs": round(tf, 2), "peak": FP16_MFMA_PEAK_TFLOPS, "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4)}
    return ro


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_cpu_baseline(w, seconds):
    """The oracle as it stands, on the host cores: one layer of the same
    workload, the same step (append T rows through the oracle codec, exact
    fp64 attention of the T query rows) on a bounded sample of (session,
    query row, Q head) items, once on one thread and once on all of them.
    Returns the same effective-GB/s unit."""
    import numpy as np

    import oracle
    t_fill = time.perf_counter()
    ref = oracle.OracleCache(w.B, w.Hkv, w.hd, w.capacity(), w.window, w.ring_step, fmt=w.fmt)
    for counts, starts, T in w.prefill_pieces():
        k, v = w.kv_block(counts, starts, T)
        ref.append(k, v, counts)
    t_fill = time.perf_counter() - t_fill
    pre = w.pre_step_lengths()
    k, v = w.kv_block([w.T] * w.B, pre, w.T)
    q = w.q(0)
    s = w.sink_logits()
    # append: repeat (append the step's rows, roll back) for ~10% of the budget
    reps, t_app = 0, 0.0
    while reps == 0 or t_app < 0.1 * seconds:
        t0 = time.perf_counter()
        ref.append(k, v)
        t_app += time.perf_counter() - t0
        ref.truncate(pre)
        reps += 1
    ref.append(k, v)
    items = w.B * w.T * w.H
    order = np.random.default_rng(0).permutation(items)
    nmax = oracle.max_threads()

    def attention_rate(threads, budget):
        oracle.set_threads(threads)
        done, t_att = 0, 0.0
        batch = max(1, min(items, 2 * threads))
        while done == 0 or t_att < budget:
            sel = order[(np.arange(batch) + done) % items]
            t0 = time.perf_counter()
            ref.attention(q, scale=w.scale, sinks=s, sel=sel, want_lse=False)
            t_att += time.perf_counter() - t0
            done += sel.size
        return done, t_att

    d1, t1 = attention_rate(1, 0.35 * seconds)
    dn, tn = attention_rate(nmax, 0.45 * seconds)
    oracle.set_threads(nmax)
    step1 = t_app / reps + t1 * items / d1
    stepn = t_app / reps + tn * items / dn
    kv = w.kv_bytes_per_decode()
    return dict(value=kv / stepn / 1e9, unit="GB/s", cores=nmax, kind="oracle",
                single_thread_value=kv / step1 / 1e9, single_thread_step_seconds=step1,
                step_seconds=stepn, cpu_model=cpu_model(), os_cpu_count=os.cpu_count(),
                sample=f"one layer of the {w.name} workload: {reps} oracle appends of {w.B * w.T} rows "
                       f"(each rolled back; single-threaded codec), then exact fp64 attention for "
                       f"{d1} (session, query row, Q head) items on 1 thread and {dn} items on {nmax} "
                       f"threads, cycling over the step's {items}; the time per step is extrapolated "
                       f"from both (cache fill {t_fill:.1f} s, not counted)")


def workload_line(w, r, ceiling):
    vo = r["kv_bytes"] / (r["ms_step"] * 1e-3) / 1e9
    return {"value": round(vo, 2), "unit": "GB/s", "ms_per_step": round(r["ms_step"], 5),
            "steps_per_s": round(1e3 / r["ms_step"], 1),
            "append_tokens_per_s": round(w.B * w.T / (r["app_ms"] * 1e-3), 1),
            "append_ms": round(r["app_ms"], 5),
            "roofline": roofline(w, r, ceiling),
            "decode_call_attn_TFLOPs": round(w.attn_flops_per_decode() / (r["call_ms"] * 1e-3) / 1e12, 3),
            "kv_bytes_per_step": r["kv_bytes"], "layers_rotated": r["L"],
            "step_launch": ("hip graph" + (" (graph mode)" if w.rollback_keep else "")) if r["graph"] else "eager",
            "importance_call": importance_summary(w, r)}


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    from decode_attention_quantized_append_amd import workloads
    w = workloads.get(args.workload)
    r = run_gpu(w, args)
    ceiling = None if args.no_ceiling else stream_read_ceiling()
    main_line = workload_line(w, r, ceiling)
    value = main_line["value"]
    line = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_line["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE,
        "data": "synthetic (seeded; shapes and distributions of the workload, no datasets or weights)",
        "config": {"workload": w.name, "kv_format": w.fmt, "sessions": w.B, "q_heads": w.H, "kv_heads": w.Hkv,
                   "head_dim": w.hd, "query_rows": w.T, "visible_rows": int(w.visible().sum()),
                   "window": w.window, "ring_rows": w.ring_cap, "layers_rotated": r["L"],
                   "kv_footprint_bytes": r["footprint"], "kv_bytes_per_step": r["kv_bytes"],
                   "parallelism": "none (1 GPU)", "step_launch": main_line["step_launch"]},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "steps_per_s": main_line["steps_per_s"],
        "append_tokens_per_s": main_line["append_tokens_per_s"],
        "roofline": main_line["roofline"],
        "stream_read_ceiling": ceiling,
        "importance_call": main_line["importance_call"],
    }
    if r["rebase"]:
        line["ring_rebase"] = r["rebase"]
    if not args.no_others:
        import torch
        others = {}
        for name in workloads.WORKLOADS:
            if name == w.name:
                continue
            torch.cuda.empty_cache()
            wo = workloads.get(name)
            ao = argparse.Namespace(**vars(args))
            ao.steps, ao.warmup, ao.layers = args.other_steps, min(args.warmup, 10), 0
            ro = run_gpu(wo, ao)
            others[name] = workload_line(wo, ro, ceiling)
            if ro["rebase"]:
                others[name]["ring_rebase"] = ro["rebase"]
        line["other_workloads"] = others
    if not args.no_cpu_baseline:
        cb = run_cpu_baseline(w, args.cpu_seconds)
        line["cpu_baseline"] = {k: (round(v, 5) if isinstance(v, float) else v) for k, v in cb.items()}
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# profiles/: summaries of rocprofv3 runs of this script (kernel traces and the
# FETCH_SIZE / WRITE_SIZE passes), rebuilt with --summarize-profiles DIR from
# the directories the commands below write.
TRACE_WORKLOADS = ("verify", "batched", "qwen_gqa", "prime", "verify_f8", "batched_f8", "prime_f8")
TRAFFIC_WORKLOADS = ("verify", "batched", "qwen_gqa", "verify_f8", "batched_f8")
PER_STEP = ("decode_stream", "decode_prime", "decode_mfma", "combine_kernel", "combine_wave_kernel", "append_kernel",
            "set_kernel")


def trace_command(wl):
    return (f"cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d <out>/trace_{wl} -o run "
            f"-- python3 /root/repo/bench.py --workload {wl} --steps 50 --warmup 5 --no-cpu-baseline "
            f"--no-others --no-ceiling > <out>/trace_{wl}.log")


def pmc_command(counter, wl):
    if wl == "copy":
        return (f"cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {counter} -d <out>/{counter}_copy -o run "
                f"-- python3 /root/repo/bench.py --calibrate-copy 1073741824")
    return (f"cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {counter} -d <out>/{counter}_{wl} -o run "
            f"-- python3 /root/repo/bench.py --workload {wl} --steps 20 --warmup 2 --no-cpu-baseline "
            f"--no-others --no-ceiling")


SQ_WORKLOADS = ("verify", "batched", "verify_f8", "batched_f8", "prime", "prime_f8")
SQ_PASSES = (("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
              "SQ_ACTIVE_INST_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VALU"),
             ("SQ_INSTS_LDS", "SQ_WAIT_ANY", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_SCA",
              "SQ_INSTS_MFMA", "SQ_INST_CYCLES_VMEM", "SQ_ACTIVE_INST_MISC"))


def sq_command(i, wl):
    return (f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc {' '.join(SQ_PASSES[i])} "
            f"-d <out>/sq{i + 1}_{wl} -o run -- python3 /root/repo/bench.py --workload {wl} --steps 5 --warmup 1 "
            f"--layers 2 --graph off --no-cpu-baseline --no-others --no-ceiling")


def _short(n):
    import re
    n = re.sub(r"^void ", "", n)
    n = n.replace("kvq::(anonymous namespace)::", "")
    return re.sub(r"\((kvq::\w+(, int)?)\)$", "", n)


def _db(path):
    import glob
    import sqlite3
    found = glob.glob(os.path.join(path, "**", "*results.db"), recursive=True)
    if not found:
        raise FileNotFoundError(f"no rocprofv3 results.db under {path}")
    return sqlite3.connect(found[0])


def _bench_line(log):
    with open(log) as f:
        for ln in f:
            if ln.startswith('{"metric"'):
                return json.loads(ln)
    return None


def summarize_profiles(d, out_dir=None):
    import collections

    from decode_attention_quantized_append_amd import workloads as W
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    H = source_hash()
    for wl in TRACE_WORKLOADS:
        path = os.path.join(d, f"trace_{wl}")
        if not os.path.isdir(path):
            continue
        c = _db(path)
        by = collections.defaultdict(list)
        for n, s, e in c.execute("select name, start, end from kernels order by start"):
            by[_short(n)].append((e - s) / 1000.0)
        b = _bench_line(os.path.join(d, f"trace_{wl}.log"))
        steps = b["steps"] if b else 50
        L = [f"# Kernel trace: {wl} workload, bench.py", "", "Command (repo at /root/repo):", "", "```",
             trace_command(wl), "```", "",
             f"Summarized by `python3 bench.py --summarize-profiles <out>`.  Source hash of the library "
             f"sources (bench.py `source_hash`): `{H}`", "",
             f"Per-step kernels, the last {steps} dispatches of each (the event-traced eager steps come "
             f"before the batched decode calls and the graph replays; these are the replays):", "",
             "| kernel | n | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
        avg = {}
        for n, dd in sorted(by.items(), key=lambda kv: -sum(kv[1][-steps:])):
            if not any(k in n for k in PER_STEP):
                continue
            t = dd[-steps:]
            avg[n] = sum(t) / len(t)
            L.append(f"| `{n}` | {len(t)} | {avg[n]:.2f} | {min(t):.2f} | {max(t):.2f} |")
        # the eager timed steps: after max(warmup, layers) untimed steps, the
        # dispatches whose duration the bench line's kernel_ms measures
        eager = {}
        if b:
            w0 = max(b["warmup"], b["config"].get("layers_rotated", 1))
            for n, dd in by.items():
                if "decode_" in n and len(dd) >= w0 + b["steps"]:
                    eager[n] = dd[w0:w0 + b["steps"]]
        w = W.get(wl)
        dec = sum(v for k, v in avg.items() if "decode_" in k)
        com = sum(v for k, v in avg.items() if "combine" in k)
        kv = w.kv_bytes_per_decode()
        if dec <= 0:
            raise RuntimeError(f"trace_{wl}: no decode kernel among the per-step kernels {sorted(avg)}")
        L += ["", f"- algorithmic K+V bytes per decode call: {kv}",
              f"- over the traced partials kernel: {kv / (dec * 1e-6) / 1e9:.1f} GB/s "
              f"({kv / (dec * 1e-6) / 1e9 / HBM_PEAK_GBPS:.4f} of 8 TB/s); over partials + combine "
              f"({dec:.2f} + {com:.2f} us): {kv / ((dec + com) * 1e-6) / 1e9:.1f} GB/s"]
        for n, t in eager.items():
            L.append(f"- `{n}` in the eager timed steps (dispatches {w0 + 1}..{w0 + len(t)}, the ones the bench "
                     f"line's kernel_ms times): avg {sum(t) / len(t):.2f} us, min {min(t):.2f}, max {max(t):.2f}")
        if b:
            ro = b["roofline"]
            L += [f"- the same run's bench line (under the profiler): partials kernel "
                  f"{ro['kernel_ms']['mean'] * 1e3:.2f} us by the library's trace events, roofline.achieved "
                  f"{ro['achieved']} GB/s (frac {ro['frac']}); decode call {ro['call']['ms'] * 1e3:.2f} us; "
                  f"step {b['ms_per_step'] * 1e3:.2f} us; value {b['value']} GB/s"]
        if w.T * w.hpk > 32:
            fl = w.attn_flops_per_decode()
            L.append(f"- attention multiply-adds x 2 per decode call: {fl}; over the traced partials kernel: "
                     f"{fl / (dec * 1e-6) / 1e12:.1f} TFLOP/s")
        with open(os.path.join(out_dir, f"decode_{wl}_kernel_trace.md"), "w") as f:
            f.write("\n".join(L) + "\n")

    def pmc(path, last=20):
        c = _db(path)
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        for name, did, v in c.execute("select kernel_name, dispatch_id, value from counters_collection"):
            per[_short(name)][did] += v
        return {k: [v for _, v in sorted(dd.items())][-last:] for k, dd in per.items()}

    sq_rows = []
    for wl in SQ_WORKLOADS:
        if not (os.path.isdir(os.path.join(d, f"sq1_{wl}")) and os.path.isdir(os.path.join(d, f"sq2_{wl}"))):
            continue
        got = {}
        for i in (1, 2):
            c = _db(os.path.join(d, f"sq{i}_{wl}"))
            per = collections.defaultdict(lambda: collections.defaultdict(float))
            for name, cn, did, v in c.execute(
                    "select kernel_name, counter_name, dispatch_id, value from counters_collection"):
                if "decode_stream" in name or "decode_prime" in name:
                    per[(_short(name), cn)][did] += v
            for (k, cn), dd in per.items():
                last = [v for _, v in sorted(dd.items())][-5:]
                got.setdefault(k, {})[cn] = sum(last) / len(last)
        for k, g in got.items():
            sq_rows.append((wl, k, g))
    if sq_rows:
        L = ["# SQ counters of the decode partials kernel", "",
             "Commands (repo at /root/repo), two passes of eight counters per workload:", "", "```"]
        for wl in dict.fromkeys(r[0] for r in sq_rows):
            L += [sq_command(0, wl), sq_command(1, wl)]
        L += ["```", "", f"Summarized by `python3 bench.py --summarize-profiles <out>`.  Source hash: `{H}`.  "
              "Each value is the mean over the last 5 dispatches (counters summed over the device).", "",
              "| workload | kernel | waves | VALU / wave | MFMA / wave | LDS / wave | SALU / wave | "
              "VALU instr per KiB of K+V | VALU-issue share of wave cycles | wait share of wave cycles | "
              "LDS bank-conflict cycles / LDS-active cycles |",
              "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
        for wl, k, g in sq_rows:
            wv = g.get("SQ_WAVES", 0) or 1
            kib = W.get(wl).kv_bytes_per_decode() / 1024
            L.append(f"| {wl} | `{k}` | {wv:.0f} | {g.get('SQ_INSTS_VALU', 0) / wv:.0f} | "
                     f"{g.get('SQ_INSTS_MFMA', 0) / wv:.0f} | {g.get('SQ_INSTS_LDS', 0) / wv:.0f} | "
                     f"{g.get('SQ_INSTS_SALU', 0) / wv:.0f} | {g.get('SQ_INSTS_VALU', 0) / kib:.1f} | "
                     f"{g.get('SQ_ACTIVE_INST_VALU', 0) / max(1, g.get('SQ_WAVE_CYCLES', 1)):.3f} | "
                     f"{g.get('SQ_WAIT_INST_ANY', 0) / max(1, g.get('SQ_WAVE_CYCLES', 1)):.3f} | "
                     f"{g.get('SQ_LDS_BANK_CONFLICT', 0) / max(1, g.get('SQ_ACTIVE_INST_LDS', 1)):.3f} |")
        L += ["", "Raw means:", "", "| workload | counter | value |", "|---|---|---:|"]
        for wl, k, g in sq_rows:
            for cn in sorted(g):
                L.append(f"| {wl} | {cn} | {g[cn]:.4g} |")
        with open(os.path.join(out_dir, "decode_sq_counters.md"), "w") as f:
            f.write("\n".join(L) + "\n")

    if not os.path.isdir(os.path.join(d, "FETCH_SIZE_copy")):
        return
    fc = pmc(os.path.join(d, "FETCH_SIZE_copy"), 10)
    wc = pmc(os.path.join(d, "WRITE_SIZE_copy"), 10)
    ck = [k for k in fc if "copy" in k.lower()][0]
    fetch_kib = sum(fc[ck]) / len(fc[ck])
    write_kib = sum(wc[ck]) / len(wc[ck])
    ff, wf = round(1048576 / fetch_kib, 3), round(1048576 / write_kib, 3)
    res = {"source_hash": H, "fetch_factor": ff, "write_factor": wf, "workloads": {}}
    rows = []
    for wl in TRAFFIC_WORKLOADS:
        if not os.path.isdir(os.path.join(d, f"FETCH_SIZE_{wl}")):
            continue
        f_ = pmc(os.path.join(d, f"FETCH_SIZE_{wl}"))
        wr = pmc(os.path.join(d, f"WRITE_SIZE_{wl}"))
        ks = {}
        for k in f_:
            if "decode_" in k or "combine" in k:
                fb = sum(f_[k]) / len(f_[k]) * 1024 * ff
                wb = sum(wr[k]) / len(wr[k]) * 1024 * wf
                ks[k] = {"fetch_bytes": fb, "write_bytes": wb}
                rows.append((wl, k, fb, wb))
        kv = W.get(wl).kv_bytes_per_decode()
        call = sum(v["fetch_bytes"] + v["write_bytes"] for v in ks.values())
        res["workloads"][wl] = {"kv_bytes": kv, "kernels": ks, "call_bytes": call}
    with open(os.path.join(out_dir, "decode_traffic.json"), "w") as f:
        json.dump(res, f, indent=1)
    L = ["# HBM traffic of the decode call (partials kernel + combine kernel)", "",
         "Commands (repo at /root/repo), one counter per run:", "", "```"]
    for wl in list(res["workloads"]) + ["copy"]:
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            L.append(pmc_command(cn, wl))
    L += ["```", "", f"Summarized by `python3 bench.py --summarize-profiles <out>`.  Source hash: `{H}`", "",
          f"Calibration: a 1 GiB device-to-device copy (`{ck}`, reads 1 GiB, writes 1 GiB) reads FETCH_SIZE = "
          f"{fetch_kib:.0f} KiB and WRITE_SIZE = {write_kib:.0f} KiB per dispatch, so FETCH_SIZE is scaled by "
          f"{ff:.3f} and WRITE_SIZE by {wf:.3f}.", "",
          "Per decode call, averaged over the last 20 dispatches of each kernel (scaled bytes):", "",
          "| workload | kernel | fetch MB | write MB |", "|---|---|---:|---:|"]
    for wl, k, fb, wb in rows:
        L.append(f"| {wl} | `{k}` | {fb / 1e6:.3f} | {wb / 1e6:.3f} |")
    L += ["", "| workload | algorithmic K+V MB | measured call MB | ratio | partials-kernel fetch / algorithmic |",
          "|---|---:|---:|---:|---:|"]
    for wl, v in res["workloads"].items():
        dfetch = sum(x["fetch_bytes"] for k, x in v["kernels"].items() if "decode_" in k)
        L.append(f"| {wl} | {v['kv_bytes'] / 1e6:.3f} | {v['call_bytes'] / 1e6:.3f} | "
                 f"{v['call_bytes'] / v['kv_bytes']:.3f} | {dfetch / v['kv_bytes']:.3f} |")
    L += ["", "The excess over the algorithmic bytes is the split-K partials (written by the partials kernel, "
          "read by the combine), the query rows, the outputs and the rows of a chunk's last tile read past "
          "its end."]
    with open(os.path.join(out_dir, "decode_hbm_traffic.md"), "w") as f:
        f.write("\n".join(L) + "\n")


if __name__ == "__main__":
    main()
