"""bench.py's rocprofv3 summaries (`--summarize-profiles`) on a synthetic
kernel-trace database: the per-step averages over the last dispatches (the
graph replays), the eager timed steps' dispatches (the ones the bench line's
kernel_ms times: after max(warmup, layers) untimed steps) and the algorithmic
bandwidth over the traced partials kernel."""
import json
import os
import sqlite3

import bench

DECODE = "void kvq::(anonymous namespace)::stream::decode_stream<4, 2, false, 2, 1, 2, false>(kvq::DecodeParams)"
COMBINE = "void kvq::(anonymous namespace)::combine_kernel<1024>(kvq::DecodeParams)"


def test_trace_summary_averages(tmp_path):
    d = tmp_path / "prof"
    (d / "trace_verify" / "host").mkdir(parents=True)
    db = sqlite3.connect(d / "trace_verify" / "host" / "run_results.db")
    db.execute("create table kernels (name text, start int, end int)")
    warmup, layers, steps, reps = 5, 3, 50, 17
    n = max(warmup, layers) + steps + reps * layers + warmup + steps
    t = 0
    for i in range(n):
        eager = max(warmup, layers) <= i < max(warmup, layers) + steps
        dur = 120_000 if eager else 100_000          # ns: the eager timed steps take 120 us
        db.execute("insert into kernels values (?, ?, ?)", (DECODE, t, t + dur))
        t += dur + 1000
        db.execute("insert into kernels values (?, ?, ?)", (COMBINE, t, t + 5000))
        t += 6000
    db.commit()
    line = {"metric": "m", "value": 1.0, "steps": steps, "warmup": warmup, "ms_per_step": 0.2,
            "config": {"layers_rotated": layers},
            "roofline": {"kernel_ms": {"mean": 0.125}, "achieved": 1.0, "frac": 0.1, "call": {"ms": 0.13}}}
    (d / "trace_verify.log").write_text(json.dumps(line) + "\n")
    out = tmp_path / "profiles"
    out.mkdir()
    bench.summarize_profiles(str(d), out_dir=str(out))
    text = (out / "decode_verify_kernel_trace.md").read_text()
    # the last 50 dispatches are the replays (100 us), the eager ones 120 us
    assert "| `stream::decode_stream<4, 2, false, 2, 1, 2, false>` | 50 | 100.00 |" in text
    assert "dispatches 6..55, the ones the bench line's kernel_ms times): avg 120.00 us" in text
    kv = 486539264
    assert f"{kv / 100e-6 / 1e9:.1f} GB/s" in text
    assert os.listdir(out) == ["decode_verify_kernel_trace.md"]
