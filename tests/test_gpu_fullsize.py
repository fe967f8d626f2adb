"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic split plan), on sampled outputs the oracle computes
one by one, and sampled rows of the planes byte by byte.

Each test brings an empty cache to the pre-step state with the same setup
appends the benchmark uses, runs one step (append T rows, decode T rows; the
verify workload then rolls back to len+3 and runs a second step) and checks.
"""
import numpy as np
import pytest

from decode_attention_quantized_append_amd import workloads

pytestmark = pytest.mark.gpu

from gpu_pair import Pair  # noqa: E402


def sampled(w, rng, n=48):
    total = w.B * w.T * w.H
    pick = set(rng.choice(total, size=min(n, total), replace=False).tolist())
    pick |= {total - 1, 0, (w.T - 1) * w.H}          # the last row of session 0 and of the last session
    return sorted(pick)


def sampled_rows(pair, rng, n=64):
    live = int((pair.ref.len - pair.ref.base).min())
    r = set(rng.choice(live, size=min(n, live), replace=False).tolist())
    return sorted(r | {0, live - 1})


def setup(name):
    w = workloads.get(name)
    p = Pair(w.B, w.H, w.Hkv, w.hd, w.capacity(extra_steps=2), w.window, w.ring_step, io=w.io_dtype)
    for counts, starts, T in w.prefill_pieces():
        k, v = w.kv_block(counts, starts, T)
        p.append(k, v, counts)
    return w, p


def step(w, p, i):
    L = p.ref.len.copy()
    k, v = w.kv_block([w.T] * w.B, L, w.T)
    p.append(k, v)
    return w.q(i), w.sink_logits()


@pytest.mark.parametrize("name", ["tiny", "qwen_gqa", "batched", "sink_ring", "verify", "prime"])
def test_full_size(name):
    rng = np.random.default_rng(7)
    w, p = setup(name)
    q, s = step(w, p, 0)
    p.check_mirror()
    assert (p.ref.len == w.lengths()).all()
    p.check_planes(rows=sampled_rows(p, rng))
    p.decode(q, w.scale, sinks=s, sel=sampled(w, rng), what=name)
    if w.rollback_keep:
        keep = p.ref.len - w.T + w.rollback_keep
        p.truncate(keep)
        p.check_mirror()
        q, s = step(w, p, 1)
        p.check_planes(rows=sampled_rows(p, rng))
        p.decode(q, w.scale, sinks=s, sel=sampled(w, rng), what=name + " after rollback")


def test_alternative_kv_distribution_reading():
    """The batched and verify shapes with the other reading of "k/v as config
    1": outlier channels x8 and v std 0.5 (scaled-down lengths)."""
    rng = np.random.default_rng(8)
    for name, over in (("batched", dict(ragged=(100, 3000))), ("verify", dict(cached=4000))):
        w = workloads.get(name, kv_dist="outlier", **over)
        p = Pair(w.B, w.H, w.Hkv, w.hd, w.capacity(), w.window, w.ring_step, io=w.io_dtype)
        for counts, starts, T in w.prefill_pieces():
            k, v = w.kv_block(counts, starts, T)
            p.append(k, v, counts)
        q, s = step(w, p, 0)
        p.check_planes()
        p.decode(q, w.scale, sinks=s, sel=sampled(w, rng, 96), what=name + " outliers")
