"""Benchmark: append + decode attention over a quantized KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--layers L] [--no-cpu-baseline] [--no-others]

A step is one pass of the whole hot path over one layer cache: the fused
quantize-and-append of T rows per session, the split-K decode plus the
log-sum-exp combine of the T query rows, and the step's length bookkeeping
(truncate back to the steady length, or the verify rollback to len+3).
Steps rotate over L independent layer caches so that the KV footprint exceeds
the 256 MB MALL and the reads come from HBM.  Inputs are seeded synthetic
tensors already resident on the GPU before timing starts.

Prints ONE JSON line.  ``value`` is the effective KV read bandwidth of the
whole step (algorithmic K+V bytes the decode must read / wall time per step).
``roofline`` reports the decode call (decode kernel + combine kernel), timed
with HIP events on the stream the library launches on, against the 8 TB/s HBM
peak; its ``traffic`` is the HBM bytes per decode call that the committed
rocprofv3 counter passes measured (profiles/decode_traffic.json), reported only
while the kernel sources still hash to the measured state.  ``cpu_baseline``
times the CPU oracle on a bounded sample of the same workload.
``other_workloads`` repeats the GPU measurement (fewer steps, no CPU
baseline) for every other workload: the batched serving tick and the
131072-row verify are the long-context shapes, tiny and the sink ring are
launch-bound.
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

HBM_PEAK_GBPS = 8000.0
METRIC = "decode attn effective KV GB/s (% of HBM peak) + steps/s; append tokens/s"
MALL_BYTES = 256 << 20


def source_hash() -> str:
    """sha256 (first 16 hex) over the kernel and host-library sources, in name order."""
    import hashlib
    d = os.path.join(ROOT, "decode_attention_quantized_append_amd", "csrc")
    h = hashlib.sha256()
    for n in sorted(os.listdir(d)):
        if n.endswith((".hip", ".cpp", ".h")):
            h.update(n.encode())
            with open(os.path.join(d, n), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per decode call (decode + combine kernels) from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE passes, scaled by the copy calibration;
    None when the sources changed since the counters were taken."""
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
    ap.add_argument("--workload", default="qwen_gqa")
    ap.add_argument("--layers", type=int, default=0)
    ap.add_argument("--split-rows", type=int, default=0)
    ap.add_argument("--tiling", default="", metavar="KERNEL,HEAD_GROUP[,SUB]",
                    help="decode kernel (1 per-head, 3 stream), KV heads per "
                         "workgroup and sub_tiles, as kvq_set_decode_tiling; default: the "
                         "library's choice")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the summary of the other workloads (each timed after the "
                         "main one, with --other-steps steps)")
    ap.add_argument("--other-steps", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--graph", choices=("auto", "on", "off"), default="auto",
                    help="replay each step as one captured HIP graph (auto and on: every "
                         "workload; verify rounds, whose lengths grow, in graph mode)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES, 10 times "
                         "(reference for scaling HBM traffic counters)")
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


def build_layers(w, L, dev, split_rows, tiling="", grow_rows=8 * 1024, graph_mode=False):
    import torch

    from decode_attention_quantized_append_amd import KvqLayerCache
    cap = w.capacity(extra_steps=0) if w.ring_cap else int(w.lengths().max()) + grow_rows
    caches = [KvqLayerCache(w.B, w.H, w.Hkv, w.hd, cap, w.window, w.ring_step, device=dev) for _ in range(L)]
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


def run_gpu(w, args):
    import torch
    dev = torch.device("cuda:0")
    L = args.layers or default_layers(w)
    # verify rounds keep rollback_keep rows each: the planes are sized to the
    # rows this run adds (eager and replayed rounds), so that graph-mode plans
    # cover little more than the real lengths
    growing = bool(w.rollback_keep)
    rounds = -(-2 * (args.warmup + args.steps) // L) + 10
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

    # Pre-bound C calls: the timed loop does no Python work beyond three calls.
    import ctypes
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
        li = i % L
        h = caches[li].h
        if ev is not None:
            ev[0].record()
        check(lib.kvq_append(h, kp, vp, dt, T, None, st), "append")
        if ev is not None:
            ev[1].record()
        check(lib.kvq_decode(h, qp, dt, T, sink_ptr, scale, op, lp, ws_ptr, ws_bytes, st), "decode")
        if ev is not None:
            ev[2].record()
        if w.rollback_keep:                        # verify: keep rollback_keep of the T rows
            check(lib.kvq_rollback(h, drop_arr, st), "rollback")
        else:                                      # steady length: drop the step's rows (a ring
            check(lib.kvq_truncate(h, pre_arr, st), "truncate")   # keeps its window resident)

    # steady workloads replay the same lengths; verify rounds grow them, which
    # graph mode (plans for every length) and the relative rollback allow
    use_graph = args.graph != "off"

    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize(dev)
    # per-call times (HIP events between the library calls of eager steps)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(args.warmup + i, events[i])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    app_ms = [e[0].elapsed_time(e[1]) for e in events]
    dec_ms = [e[1].elapsed_time(e[2]) for e in events]
    if use_graph:
        # one graph per layer for the whole step; the per-call times stay those
        # of the eager steps above (HIP events between the library calls)
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
        if growing:   # the replays moved the device lengths: bring the host mirrors back in step
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
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        check(lib.kvq_append(h, kp, vp, dt, T, None, stream), "append")
        check(lib.kvq_decode(h, qp, dt, T, sink_ptr, scale, op, lp, ws_ptr, ws_bytes, stream), "decode")
        e0.record()
        check(lib.kvq_importance(h, qp, dt, T, scale, lp, imp.data_ptr(), stream), "importance")
        e1.record()
        if w.rollback_keep:
            check(lib.kvq_rollback(h, drop_arr, stream), "rollback")
        else:
            check(lib.kvq_truncate(h, pre_arr, stream), "truncate")
        torch.cuda.synchronize(dev)
        imp_ms.append(e0.elapsed_time(e1))
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
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            base0 = caches[li].host_lengths()[1][0]
            e0.record()
            check(lib.kvq_append(h, kp, vp, dt, T, one, stream), "append with rebase")
            e1.record()
            torch.cuda.synchronize(dev)
            assert caches[li].host_lengths()[1][0] > base0, "the append did not rebase"
            times.append(e0.elapsed_time(e1))
        ln, bs = caches[0].host_lengths()
        rebase = dict(append_with_rebase_ms=round(sum(times) / len(times), 5),
                      rows_moved_per_session=int(ln[0] - 1 - bs[0]), ring_step=w.ring_step,
                      amortized_ms_per_append=round((sum(times) / len(times) - sum(app_ms) / len(app_ms))
                                                    / w.ring_step, 6))
    kv_bytes = w.kv_bytes_per_decode()
    ms_step = wall * 1e3 / args.steps
    dec_avg = sum(dec_ms) / len(dec_ms)
    app_avg = sum(app_ms) / len(app_ms)
    dec_sorted = sorted(dec_ms)
    return dict(L=L, cap=cap, ms_step=ms_step, graph=use_graph, dec_ms=dec_avg, app_ms=app_avg, rebase=rebase,
                imp_ms=sum(imp_ms) / len(imp_ms),
                dec_p10=dec_sorted[len(dec_ms) // 10], dec_p90=dec_sorted[(9 * len(dec_ms)) // 10],
                kv_bytes=kv_bytes, ws_bytes=ws_bytes,
                footprint=L * (caches[0].sizes.k_planes_bytes + caches[0].sizes.v_planes_bytes))


def importance_summary(w, r):
    """The importance pass reads the K rows of the step's span once."""
    kbytes = int(w.span().sum()) * w.k_row_bytes
    return {"ms": round(r["imp_ms"], 5), "k_bytes": kbytes,
            "GBps": round(kbytes / (r["imp_ms"] * 1e-3) / 1e9, 2)}


def run_cpu_baseline(w, seconds):
    """The oracle as it stands, on the host cores: one layer, the same step
    (append T rows through the oracle codec, exact attention of the T query
    rows), on a bounded sample of (session, row, head) items when a whole
    step would take too long.  Returns the same effective-GB/s unit."""
    import numpy as np

    import oracle
    ref = oracle.OracleCache(w.B, w.Hkv, w.hd, w.capacity(), w.window, w.ring_step)
    for counts, starts, T in w.prefill_pieces():
        k, v = w.kv_block(counts, starts, T)
        ref.append(k, v, counts)
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
    # attention: cycle over the step's (session, query row, Q head) items for the rest
    items = w.B * w.T * w.H
    order = np.random.default_rng(0).permutation(items)
    done, t_att = 0, 0.0
    batch = max(1, min(items, 8 * oracle.max_threads()))
    while done == 0 or t_att < 0.9 * seconds:
        sel = order[(np.arange(batch) + done) % items]
        t0 = time.perf_counter()
        ref.attention(q, scale=w.scale, sinks=s, sel=sel, want_lse=False)
        t_att += time.perf_counter() - t0
        done += sel.size
    step_s = t_app / reps + t_att * items / done
    return dict(value=w.kv_bytes_per_decode() / step_s / 1e9, unit="GB/s", cores=oracle.max_threads(),
                kind="oracle",
                sample=f"one layer of the same workload: {reps} oracle appends of {w.B * w.T} rows "
                       f"(each rolled back) and exact attention for {done} (session, query row, Q head) "
                       f"items cycling over the step's {items}; time per step extrapolated from both",
                step_seconds=step_s)


def main():
    args = parse()
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
    value = r["kv_bytes"] / (r["ms_step"] * 1e-3) / 1e9
    achieved = r["kv_bytes"] / (r["dec_ms"] * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; shapes and distributions of the workload, no datasets or weights)",
        "config": {"workload": w.name, "sessions": w.B, "q_heads": w.H, "kv_heads": w.Hkv,
                   "head_dim": w.hd, "query_rows": w.T, "visible_rows": int(w.visible().sum()),
                   "window": w.window, "ring_rows": w.ring_cap, "layers_rotated": r["L"],
                   "kv_footprint_bytes": r["footprint"], "kv_bytes_per_step": r["kv_bytes"],
                   "parallelism": "none (1 GPU)", "step_launch": ("hip graph" + (" (graph mode)" if w.rollback_keep else "")) if r["graph"] else "eager"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "steps_per_s": round(1e3 / r["ms_step"], 1),
        "append_tokens_per_s": round(w.B * w.T / (r["app_ms"] * 1e-3), 1),
        "decode_call_ms": {"mean": round(r["dec_ms"], 5), "p10": round(r["dec_p10"], 5),
                           "p90": round(r["dec_p90"], 5)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(w.name), "traffic_unit": "bytes per decode call",
                     "algorithmic": r["kv_bytes"],
                     "kernel": "kvq_decode call (split-K partials kernel + LSE combine kernel), HIP events"},
    }
    line["importance_call"] = importance_summary(w, r)
    if r["rebase"]:
        line["ring_rebase"] = r["rebase"]
    if not args.no_others:
        # the other workloads, same step and measurement, fewer steps; each
        # is a parity case of the tests as well
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
            vo = ro["kv_bytes"] / (ro["ms_step"] * 1e-3) / 1e9
            ac = ro["kv_bytes"] / (ro["dec_ms"] * 1e-3) / 1e9
            others[name] = {
                "value": round(vo, 2), "unit": "GB/s", "ms_per_step": round(ro["ms_step"], 5),
                "steps_per_s": round(1e3 / ro["ms_step"], 1),
                "append_tokens_per_s": round(wo.B * wo.T / (ro["app_ms"] * 1e-3), 1),
                "decode_call_ms": round(ro["dec_ms"], 5), "decode_call_GBps": round(ac, 2),
                "decode_call_frac_hbm_peak": round(ac / HBM_PEAK_GBPS, 4),
                "decode_call_attn_TFLOPs": round(wo.attn_flops_per_decode() / (ro["dec_ms"] * 1e-3) / 1e12, 3),
                "kv_bytes_per_step": ro["kv_bytes"], "layers_rotated": ro["L"],
                "steps": ao.steps, "step_launch": ("hip graph" + (" (graph mode)" if wo.rollback_keep else "")) if ro["graph"] else "eager",
                "traffic": measured_traffic(name)}
            others[name]["importance_call"] = importance_summary(wo, ro)
            if ro["rebase"]:
                others[name]["ring_rebase"] = ro["rebase"]
        line["other_workloads"] = others
    if not args.no_cpu_baseline:
        cb = run_cpu_baseline(w, args.cpu_seconds)
        line["cpu_baseline"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in cb.items()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
