"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic split plan): every live byte of the K and V planes
against the oracle's, and every output and log-sum-exp element against the
oracle's exact attention.

Each test brings an empty cache to the pre-step state with the same setup
appends the benchmark uses, runs one step (append T rows, decode T rows; the
verify workload then rolls back to len+3 and runs a second step) and checks.
"""
import pytest

from decode_attention_quantized_append_amd import workloads

pytestmark = pytest.mark.gpu

from gpu_pair import Pair  # noqa: E402


def setup(name):
    w = workloads.get(name)
    p = Pair(w.B, w.H, w.Hkv, w.hd, w.capacity(extra_steps=2), w.window, w.ring_step, io=w.io_dtype, fmt=w.fmt)
    for counts, starts, T in w.prefill_pieces():
        k, v = w.kv_block(counts, starts, T)
        p.append(k, v, counts)
    return w, p


def step(w, p, i):
    L = p.ref.len.copy()
    k, v = w.kv_block([w.T] * w.B, L, w.T)
    p.append(k, v)
    return w.q(i), w.sink_logits()


@pytest.mark.parametrize("name", ["tiny", "qwen_gqa", "batched", "sink_ring", "verify", "prime", "verify_f8",
                                  "batched_f8", "prime_f8"])
def test_full_size(name):
    w, p = setup(name)
    q, s = step(w, p, 0)
    p.check_mirror()
    assert (p.ref.len == w.lengths()).all()
    print(f"\ncase {name}: planes", flush=True)
    p.check_planes()
    print(f"case {name}: decode", flush=True)
    p.decode(q, w.scale, sinks=s, what=name)
    if w.rollback_keep:
        keep = p.ref.len - w.T + w.rollback_keep
        p.truncate(keep)
        p.check_mirror()
        q, s = step(w, p, 1)
        print(f"case {name}: after rollback", flush=True)
        p.check_planes()
        p.decode(q, w.scale, sinks=s, what=name + " after rollback")


def test_alternative_kv_distribution_reading():
    """The batched and verify shapes with the other reading of "k/v as config
    1": outlier channels x8 and v std 0.5 (scaled-down lengths)."""
    for name, over in (("batched", dict(ragged=(100, 3000))), ("verify", dict(cached=4000))):
        w = workloads.get(name, kv_dist="outlier", **over)
        p = Pair(w.B, w.H, w.Hkv, w.hd, w.capacity(), w.window, w.ring_step, io=w.io_dtype)
        for counts, starts, T in w.prefill_pieces():
            k, v = w.kv_block(counts, starts, T)
            p.append(k, v, counts)
        q, s = step(w, p, 0)
        p.check_planes()
        p.decode(q, w.scale, sinks=s, what=name + " outliers")
