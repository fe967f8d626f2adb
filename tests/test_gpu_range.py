"""GPU parity over the whole input range the formats allow: V blocks with
steps up to the fp16 maximum's range (block ranges to 6e4) and queries from
1e-30 to 1e5 in magnitude, bf16 and fp32, on every decode kernel and layout.

The decode multiplies each softmax weight P (at most 2^8) by a V block's
step as fp16; tiles with steps of 2^7 or more switch the P V accumulator to
units of 2^-E, and query rows are divided by a power of two before their
fp16 cast.  These tests check that against the oracle's fp64 attention.

Tolerance.  The element bound is |gpu - oracle| <= atol + 1e-2 |oracle| with
atol = 2e-3 for values of the workloads' scale (|v| up to about 4).  The
fp16 weights give an error up to about 2^-11 sum_j p_j |v_j| / sum_j p_j,
which grows with the V magnitude, so for V blocks of larger range atol is
the same bound relative to that scale: 2e-3 * max(1, max|V'| / 4).
"""
import zlib

import numpy as np
import pytest
import torch

from decode_attention_quantized_append_amd import kvq
from decode_attention_quantized_append_amd.workloads import round_bf16

pytestmark = pytest.mark.gpu

from gpu_pair import ATOL, DEV, Pair, assert_close, to_dev  # noqa: E402

# name: (B, H, Hkv, hd, T, lengths, window, io, tiling)
SHAPES = {
    "hd128_gqa": (2, 32, 8, 128, 1, [700, 300], 0, "bf16", None),
    "hd128_long_rowstreams": (2, 40, 8, 128, 1, [3000, 1700], 0, "bf16", None),
    "hd256_verify_dimhalves": (1, 16, 4, 256, 8, [600], 0, "bf16", None),
    "hd128_T8_dimhalves_f32": (2, 16, 4, 128, 8, [500, 90], 0, "f32", None),
    "hd64_rowgroups": (2, 24, 1, 64, 1, [400, 77], 0, "bf16", (kvq.KVQ_DECODE_STREAM, 0, 2)),
    "hd256_rowtiles": (1, 16, 4, 256, 8, [300], 0, "bf16", (kvq.KVQ_DECODE_STREAM, 0, 1)),
    "hd96_perhead": (2, 6, 2, 96, 2, [300, 41], 50, "f32", None),
    "hd128_perhead_T8": (1, 32, 8, 128, 8, [333], 0, "bf16", (kvq.KVQ_DECODE_PER_HEAD, 0, 0)),
    "hd256_perhead_T8": (1, 16, 4, 256, 8, [260], 0, "bf16", (kvq.KVQ_DECODE_PER_HEAD, 0, 0)),
    "hd128_prime_T40": (2, 32, 8, 128, 40, [500, 90], 0, "bf16", (kvq.KVQ_DECODE_PRIME, 0, 0)),
    "hd64_prime_T70_window": (1, 16, 4, 64, 70, [400], 100, "bf16", None),
}


def big_v_rows(rng, B, n, Hkv, hd, mode):
    """V rows whose 32-element blocks have ranges from about 1 to 6e4.
    mixed: each row picks a magnitude class (N(0,1), range 1e3, 5e3 (step
    about 160), 3e4 (step about 970)); all: every block spans about 6e4
    (step about 1900, the largest shift)."""
    if mode == "all":
        v = rng.uniform(-3e4, 3e4, size=(B, n, Hkv, hd))
    else:
        cls = rng.integers(0, 4, size=(B, n, 1, 1))
        amp = np.choose(cls, [1.0, 500.0, 2500.0, 15000.0])
        v = rng.uniform(-1.0, 1.0, size=(B, n, Hkv, hd)) * amp
        v = np.where(cls == 0, rng.standard_normal((B, n, Hkv, hd)), v)
    return v.astype(np.float32)


def fill(p, rng, lens, v_mode=None, io="bf16"):
    B, Hkv, hd = p.B, p.Hkv, p.hd
    lens = np.asarray(lens)
    done = np.zeros(B, np.int64)
    while np.any(done < lens):
        n = np.minimum(lens - done, 400)
        m = int(n.max())
        k = rng.standard_normal((B, m, Hkv, hd)).astype(np.float32)
        v = big_v_rows(rng, B, m, Hkv, hd, v_mode) if v_mode else rng.standard_normal((B, m, Hkv, hd)).astype(np.float32)
        if io == "bf16":
            k, v = round_bf16(k), round_bf16(v)
        p.append(k, v, n.tolist())
        done += n


def v_scale_atol(p):
    """2e-3 relative to the workloads' |v| scale of about 4 (module doc);
    max|v| of the appended rows, 5 % added for the q5_1 rounding."""
    return ATOL * max(1.0, 1.05 * p.vmax / 4.0)


@pytest.mark.parametrize("v_mode", ["mixed", "all"])
@pytest.mark.parametrize("name", sorted(SHAPES))
def test_decode_large_v_steps(name, v_mode):
    B, H, Hkv, hd, T, lens, window, io, tiling = SHAPES[name]
    rng = np.random.default_rng(zlib.crc32(f"{name}/{v_mode}".encode()))
    p = Pair(B, H, Hkv, hd, max(lens) + 8, window, 0, io=io)
    if tiling:
        p.gpu.set_decode_tiling(*tiling)
    fill(p, rng, lens, v_mode, io)
    q = rng.standard_normal((B, T, H, hd)).astype(np.float32)
    q = round_bf16(q) if io == "bf16" else q
    s = rng.standard_normal(H).astype(np.float32) if hd == 96 else None
    print(f"\ncase {name} v={v_mode}", flush=True)
    p.decode(q, float(np.float32(1 / np.sqrt(hd))), sinks=s, what=f"{name} v={v_mode}", atol=v_scale_atol(p))


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_decode_large_and_tiny_k_steps(name):
    """K blocks over the q8_0 range: in session 0 each row takes N(0,1),
    uniform +-3e4 (step about 236) or uniform +-6e4 (step about 472, above
    2^8) blocks, with queries of 3e-4 N(0,1) so that scores stay near 10; in
    session 1 each row takes N(0,1) or 1e-6 N(0,1) blocks (subnormal fp16
    steps) with N(0,1) queries.  Checks every kernel's K products (exact
    codes times steps, or the exact fp16 pairs of the prime kernel, with its
    shift for steps of 2^8 and more) against the oracle."""
    B, H, Hkv, hd, T, lens, window, io, tiling = SHAPES[name]
    B = 2
    lens = (list(lens) + [lens[0]])[:2]
    rng = np.random.default_rng(zlib.crc32(f"{name}/k".encode()))
    p = Pair(B, H, Hkv, hd, max(lens) + 8, window, 0, io=io)
    if tiling:
        p.gpu.set_decode_tiling(*tiling)
    lens = np.asarray(lens)
    done = np.zeros(B, np.int64)
    while np.any(done < lens):
        n = np.minimum(lens - done, 400)
        m = int(n.max())
        k = rng.standard_normal((B, m, Hkv, hd))
        cls = rng.integers(0, 3, size=(m, Hkv, 1))
        k[0] = np.where(cls == 1, rng.uniform(-3e4, 3e4, (m, Hkv, hd)), k[0])
        k[0] = np.where(cls == 2, rng.uniform(-6e4, 6e4, (m, Hkv, hd)), k[0])
        k[1] = np.where(cls == 1, k[1] * 1e-6, k[1])
        k = k.astype(np.float32)
        v = rng.standard_normal((B, m, Hkv, hd)).astype(np.float32)
        if io == "bf16":
            k, v = round_bf16(k), round_bf16(v)
        p.append(k, v, n.tolist())
        done += n
    q = rng.standard_normal((B, T, H, hd))
    q[0] *= 3e-4
    q = q.astype(np.float32)
    q = round_bf16(q) if io == "bf16" else q
    print(f"\ncase {name} k range", flush=True)
    p.decode(q, float(np.float32(1 / np.sqrt(hd))), what=f"{name} k range")


def extreme_q(rng, B, T, H, hd, io, big=1e5, spike_at=1e4):
    """Query rows of very different magnitudes: x big, x1e-6 (below fp16's
    normal range), x1e-30, all zero, one element spike_at among tiny ones
    (dim 3), and N(0,1); the classes are mixed within every group of rows."""
    q = rng.standard_normal((B, T, H, hd)).astype(np.float64)
    cls = rng.integers(0, 6, size=(B, T, H, 1))
    q = np.where(cls == 0, q * big, q)
    q = np.where(cls == 1, q * 1e-6, q)
    q = np.where(cls == 2, q * 1e-30, q)
    q = np.where(cls == 3, 0.0, q)
    spike = np.zeros_like(q)
    spike[..., 3] = spike_at
    q = np.where(cls == 4, q * 1e-3 + spike, q)
    q = q.astype(np.float32)
    return round_bf16(q) if io == "bf16" else q


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("name", sorted(SHAPES))
def test_decode_extreme_queries(name, io):
    B, H, Hkv, hd, T, lens, window, _, tiling = SHAPES[name]
    rng = np.random.default_rng(zlib.crc32(f"{name}/{io}/q".encode()))
    p = Pair(B, H, Hkv, hd, max(lens) + 8, window, 0, io=io)
    if tiling:
        p.gpu.set_decode_tiling(*tiling)
    fill(p, rng, lens, None, io)
    q = extreme_q(rng, B, T, H, hd, io)
    print(f"\ncase {name} q={io}", flush=True)
    p.decode(q, float(np.float32(1 / np.sqrt(hd))), what=f"{name} extreme q {io}")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_importance_extreme_queries(io):
    """Importance recomputes each score in fp32 and forms exp(s - lse), so
    its relative accuracy is that of fp32 scores: scores of magnitude 1e5
    carry absolute errors near 1e-2.  The query range of the fp16 cast is
    covered here with moderate scores: a 1e5 element sits on a K dimension
    that is zero in every key, next to rows of 1e2, 1e-6, 1e-30 and 0."""
    rng = np.random.default_rng(5 if io == "bf16" else 6)
    B, H, Hkv, hd, T = 2, 16, 4, 128, 4
    p = Pair(B, H, Hkv, hd, 520, 0, 0, io=io)
    lens = np.asarray([500, 260])
    done = np.zeros(B, np.int64)
    while np.any(done < lens):
        n = np.minimum(lens - done, 400)
        m = int(n.max())
        k = rng.standard_normal((B, m, Hkv, hd)).astype(np.float32)
        k[..., 3] = 0.0
        v = rng.standard_normal((B, m, Hkv, hd)).astype(np.float32)
        if io == "bf16":
            k, v = round_bf16(k), round_bf16(v)
        p.append(k, v, n.tolist())
        done += n
    q = extreme_q(rng, B, T, H, hd, io, big=1e2, spike_at=1e5)
    scale = float(np.float32(1 / np.sqrt(hd)))
    qd = to_dev(q, io)
    out, lse = p.gpu.decode(qd, scale)
    imp = p.gpu.importance(qd, scale, lse)
    torch.cuda.synchronize(DEV)
    want = p.ref.importance(q, scale=scale)
    assert_close(imp.cpu().numpy(), want, f"importance extreme q {io}")
