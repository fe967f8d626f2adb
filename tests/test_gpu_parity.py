"""GPU parity: the HIP path through the C ABI against the oracle, element by
element, on seeded inputs at sizes the oracle finishes in seconds that still
span several 64-row tiles, several split-K chunks and ragged tails.

Codes and scales must be bit-exact; attention outputs and log-sum-exps must
satisfy |gpu - oracle| <= 2e-3 + 1e-2 |oracle| for every element.
"""
import numpy as np
import pytest
import torch

from decode_attention_quantized_append_amd import KvqError, kvq
from decode_attention_quantized_append_amd.workloads import round_bf16

pytestmark = pytest.mark.gpu

from gpu_pair import DEV, Pair, assert_close, to_dev  # noqa: E402


def rows(rng, B, T, Hkv, hd, io="bf16", scale=1.0, outliers=False):
    k = rng.standard_normal((B, T, Hkv, hd)).astype(np.float32) * scale
    v = rng.standard_normal((B, T, Hkv, hd)).astype(np.float32) * scale
    if outliers:
        for g in range(Hkv):
            k[:, :, g, rng.choice(hd, 4, replace=False)] *= 8.0
        v *= 0.5
    return (round_bf16(k), round_bf16(v)) if io == "bf16" else (k, v)


def qrows(rng, B, T, H, hd, io="bf16"):
    q = rng.standard_normal((B, T, H, hd)).astype(np.float32)
    return round_bf16(q) if io == "bf16" else q


# -- append: codes bit-exact -------------------------------------------------------
@pytest.mark.parametrize("B,Hkv,hd,io", [(1, 1, 64, "f32"), (1, 8, 128, "bf16"), (3, 8, 128, "bf16"),
                                         (4, 8, 64, "bf16"), (2, 4, 256, "bf16"), (2, 3, 96, "f32"),
                                         (1, 2, 32, "f32")])
def test_append_codes_bit_exact(B, Hkv, hd, io):
    rng = np.random.default_rng(hd * 7 + B)
    p = Pair(B, 4 * Hkv, Hkv, hd, 400, io=io)
    for T, counts in [(1, None), (7, None), (64, [64 - b for b in range(B)]), (130, None), (3, [0] + [3] * (B - 1))]:
        k, v = rows(rng, B, T, Hkv, hd, io, scale=rng.choice([0.01, 1.0, 30.0]), outliers=(hd == 128))
        p.append(k, v, counts)
        p.check_mirror()
    p.check_planes()


def test_append_edge_blocks():
    """Ties at half a step, zero and constant blocks, subnormal fp16 scales,
    -0.0, a huge range and one-hot blocks: every byte equals the oracle's."""
    hd = 32 * 16
    blocks = []
    d = 0.125
    tie = np.zeros(32, np.float32)
    tie[0] = 127 * d
    tie[1:] = (np.arange(31) - 15 + 0.5) * d
    blocks.append(tie)
    blocks.append(np.zeros(32, np.float32))
    blocks.append(np.full(32, 1.5, np.float32))
    blocks.append(np.full(32, -0.0, np.float32))
    blocks.append(np.linspace(-1e-6, 1e-6, 32).astype(np.float32))           # subnormal fp16 scale
    blocks.append((np.arange(32) * 2.0 ** -24).astype(np.float32))
    blocks.append(np.linspace(-3e4, 3e4, 32).astype(np.float32))
    one = np.zeros(32, np.float32)
    one[5] = -7.0
    blocks.append(one)
    q5tie = np.zeros(32, np.float32)
    q5tie[1] = 31 * 0.25
    q5tie[2:] = (np.arange(30) + 0.5) * 0.25
    blocks.append(q5tie)
    stored_min = np.full(32, 0.1, np.float32)
    stored_min[1], stored_min[2] = 7.85, 0.4749875
    blocks.append(stored_min)
    mixed_zero = np.zeros(32, np.float32)
    mixed_zero[1::3] = -0.0
    mixed_zero[2::5] = 2.5
    blocks.append(mixed_zero)
    rng = np.random.default_rng(3)
    while len(blocks) < 16:
        blocks.append((rng.standard_normal(32) * 10.0 ** rng.integers(-5, 4)).astype(np.float32))
    row = np.concatenate(blocks).reshape(1, 1, 4, hd // 4)     # 4 KV heads of 128
    for io in ("f32", "bf16"):
        x = row if io == "f32" else round_bf16(row)
        p = Pair(1, 4, 4, hd // 4, 4, io=io)
        p.append(x, -x)
        p.append(x[:, :, :, ::-1].copy(), x)
        p.check_planes()


# -- decode parity -----------------------------------------------------------------
SMALL = {
    # name: (B, H, Hkv, hd, T, lengths, window, cap, step, sinks, io, outliers)
    "tiny": (1, 4, 1, 64, 1, [256], 0, 300, 0, False, "f32", False),
    "qwen_gqa_small": (1, 32, 8, 128, 1, [1500], 0, 1600, 0, False, "bf16", True),
    "batched_small": (16, 40, 8, 128, 1, [1, 2, 63, 64, 65, 127, 128, 129, 700, 1023, 1024, 1025,
                                          333, 900, 5, 1100], 0, 1200, 0, False, "bf16", False),
    "sink_ring_small": (4, 64, 8, 64, 1, [1000, 1000, 1000, 1000], 64, 128, 32, True, "bf16", False),
    "verify_small": (2, 16, 4, 256, 8, [600, 333], 0, 700, 0, False, "bf16", False),
    "hd32_gqa7": (2, 7, 1, 32, 3, [200, 70], 0, 256, 0, True, "f32", False),
    "hd96_window": (3, 6, 2, 96, 2, [300, 40, 2], 50, 320, 0, False, "bf16", False),
    "qwen_f32_small": (2, 32, 8, 128, 2, [900, 161], 0, 1000, 0, True, "f32", True),
    "verify_f32_small": (2, 16, 4, 256, 8, [500, 75], 0, 600, 0, True, "f32", False),
    # prompt chunks (eight and five groups of query rows: the prime kernel)
    "prime_small": (1, 32, 8, 128, 64, [700], 256, 1000, 0, True, "bf16", True),
    "prime_ring_small": (2, 8, 2, 64, 40, [600, 300], 200, 400, 32, False, "f32", False),
}


def build_small(name, seed=0):
    B, H, Hkv, hd, T, lens, window, cap, step, sinks, io, outl = SMALL[name]
    rng = np.random.default_rng(seed + len(name))
    p = Pair(B, H, Hkv, hd, cap, window, step, io=io)
    lens = np.asarray(lens)
    done = np.zeros(B, np.int64)
    piece = 64 if step else 400
    while np.any(done < lens):
        n = np.minimum(lens - done, piece)
        k, v = rows(rng, B, int(n.max()), Hkv, hd, io, outliers=outl)
        p.append(k, v, n.tolist())
        done += n
    q = qrows(rng, B, T, H, hd, io)
    s = rng.standard_normal(H).astype(np.float32) if sinks else None
    return p, q, s, float(np.float32(1 / np.sqrt(hd)))


@pytest.mark.parametrize("name", sorted(SMALL))
def test_decode_parity(name):
    p, q, s, scale = build_small(name)
    p.check_mirror()
    p.check_planes()
    p.decode(q, scale, sinks=s, what=name)


def test_decode_split_invariance():
    """Output is invariant across split plans (log-sum-exp identity)."""
    p, q, s, scale = build_small("batched_small")
    qd = to_dev(q, "bf16")
    outs = []
    for rows_ in (64, 128, 320, 1024, 0):
        p.gpu.set_split_rows(rows_)
        o, l = p.gpu.decode(qd, scale)
        outs.append((o.cpu().numpy(), l.cpu().numpy()))
    # P enters the P.V product and the row sums as fp16, rounded relative to
    # each split's own running max: outputs agree within Pair.pv_atol, the
    # log-sum-exps within Pair.lse_atol.
    for o, l in outs[1:]:
        np.testing.assert_allclose(o, outs[0][0], atol=p.pv_atol(), rtol=0)
        np.testing.assert_allclose(l, outs[0][1], atol=p.lse_atol(), rtol=0)
    p.decode(q, scale)


# Decode kernels and tilings (kernel, KV heads per workgroup, waves per KV
# head) that fit each shape; the automatic choice is covered by
# test_decode_parity.
PH, ST, PR = kvq.KVQ_DECODE_PER_HEAD, kvq.KVQ_DECODE_STREAM, kvq.KVQ_DECODE_PRIME
TILINGS = {
    "qwen_gqa_small": [(ST, 8, 0), (ST, 2, 0), (ST, 1, 0), (ST, 8, 1), (ST, 8, 2), (ST, 2, 2)],
    "batched_small": [(ST, 8, 0), (ST, 4, 0), (ST, 8, 2), (ST, 4, 2)],
    "sink_ring_small": [(ST, 8, 0), (ST, 2, 0), (ST, 8, 2)],
    "verify_small": [(ST, 4, 0), (ST, 1, 0), (ST, 4, 1), (ST, 2, 1), (ST, 1, 1), (ST, 4, 2), (ST, 2, 2),
                     (ST, 1, 2), (ST, 4, 3), (ST, 2, 3), (ST, 1, 3)],
    "qwen_f32_small": [(ST, 8, 0), (ST, 4, 0), (ST, 8, 1)],
    "tiny": [(ST, 1, 0)],
    "verify_f32_small": [(ST, 4, 1), (ST, 2, 1), (ST, 4, 2), (ST, 2, 2), (ST, 4, 3), (ST, 2, 3)],
    "prime_small": [(PR, 0, 0), (ST, 0, 0), (ST, 4, 0), (ST, 0, 3)],
    "prime_ring_small": [(PR, 0, 0), (ST, 0, 0), (ST, 2, 2)],
}


@pytest.mark.parametrize("name,kernel,gh,sub", [(n, *t) for n, lst in TILINGS.items() for t in lst])
def test_decode_tiling_parity(name, kernel, gh, sub):
    p, q, s, scale = build_small(name)
    p.gpu.set_decode_tiling(kernel, gh, sub)
    p.decode(q, scale, sinks=s, what=f"{name} kernel={kernel} gh={gh} sub={sub}")


@pytest.mark.parametrize("name", sorted(TILINGS))
def test_decode_tilings_agree(name):
    """Every kernel and tiling gives the same outputs up to the fp16 rounding
    of P (Pair.pv_atol, Pair.lse_atol)."""
    p, q, s, scale = build_small(name)
    io = SMALL[name][10]
    qd = to_dev(q, io)
    sd = torch.from_numpy(s).to(DEV) if s is not None else None
    outs = []
    for kernel, gh, sub in [(PH, 0, 0), (kvq.KVQ_DECODE_AUTO, 0, 0)] + TILINGS[name]:
        p.gpu.set_decode_tiling(kernel, gh, sub)
        for rows_ in (0, 64, 256):
            p.gpu.set_split_rows(rows_)
            o, l = p.gpu.decode(qd, scale, sinks=sd)
            outs.append((o.cpu().numpy(), l.cpu().numpy()))
    for o, l in outs[1:]:
        np.testing.assert_allclose(o, outs[0][0], atol=p.pv_atol(), rtol=0)
        np.testing.assert_allclose(l, outs[0][1], atol=p.lse_atol(), rtol=0)


@pytest.mark.parametrize("name", sorted(TILINGS))
def test_decode_plans_exact_weights(name):
    """With zero queries every visible row scores 0, so every weight is
    exactly 1 in fp16 and in fp32, and so is each weight times its q5_1 step:
    the only rounding left is the fp32 summation (and the sink's exp in the
    combine).  Every kernel, tiling and split plan must then give the mean of
    the visible V rows (with the sink in the denominator) and lse =
    log(rows + sum of the sink's exp), as the oracle does, within 1e-5 of the
    V scale: far below Pair.pv_atol, so a row dropped, counted twice or
    masked wrongly by a plan shows up at any length here."""
    p, q, s, scale = build_small(name)
    q = np.zeros_like(q)
    io = SMALL[name][10]
    qd = to_dev(q, io)
    sd = torch.from_numpy(s).to(DEV) if s is not None else None
    want, want_lse = p.ref.attention(q, scale=scale, sinks=s)
    atol = 1e-5 * max(1.0, p.vmax)
    for kernel, gh, sub in [(PH, 0, 0), (kvq.KVQ_DECODE_AUTO, 0, 0)] + TILINGS[name]:
        p.gpu.set_decode_tiling(kernel, gh, sub)
        for rows_ in (0, 64, 256):
            p.gpu.set_split_rows(rows_)
            o, l = p.gpu.decode(qd, scale, sinks=sd)
            what = f"{name} kernel={kernel} gh={gh} sub={sub} split={rows_}"
            np.testing.assert_allclose(o.cpu().numpy(), want, atol=atol, rtol=0, err_msg=what)
            np.testing.assert_allclose(l.cpu().numpy(), want_lse, atol=1e-5, rtol=0, err_msg=what)


# -- many query rows: groups of 32 / hpk rows per decode launch, one combine -------
MANY = {
    # name: (B, H, Hkv, hd, T, lengths, window, sinks, io, tiling)
    "hd128_T40_sinks": (2, 8, 2, 128, 40, [700, 300], 0, True, "bf16", None),
    "hd256_T19": (1, 16, 4, 256, 19, [500], 0, False, "bf16", None),
    "hd256_T19_rowgroups": (1, 16, 4, 256, 19, [500], 0, False, "bf16", (kvq.KVQ_DECODE_STREAM, 0, 2)),
    "hd256_T19_dimhalves": (1, 16, 4, 256, 19, [500], 0, True, "bf16", (kvq.KVQ_DECODE_STREAM, 0, 3)),
    "hd128_T40_dimhalves": (2, 8, 2, 128, 40, [700, 300], 0, True, "bf16", (kvq.KVQ_DECODE_STREAM, 0, 3)),
    "hd128_T21_window_dimhalves_f32": (2, 32, 8, 128, 21, [400, 130], 90, False, "f32", (kvq.KVQ_DECODE_STREAM, 4, 3)),
    "hd256_T13_window_dimhalves_f32": (2, 8, 2, 256, 13, [300, 97], 70, True, "f32", (kvq.KVQ_DECODE_STREAM, 2, 3)),
    "hd64_hpk1_T100": (1, 4, 4, 64, 100, [400], 0, False, "bf16", None),
    "hd64_T70_window": (2, 16, 4, 64, 70, [330, 71], 45, True, "bf16", None),
    "hd96_T33_window_f32": (2, 6, 2, 96, 33, [260, 40], 50, False, "f32", None),
    "hd128_T24_perhead_f32": (2, 32, 8, 128, 24, [300, 129], 0, True, "f32", (kvq.KVQ_DECODE_PER_HEAD, 0)),
    # the prime kernel: eight groups of query rows per workgroup sharing each
    # KV tile; partial groups (hpk 5: 30 of 32 rows), partial blocks of
    # groups, a session holding exactly the T rows, windows, fp32 queries
    "hd128_T200_prime_window_sinks": (2, 32, 8, 128, 200, [900, 260], 300, True, "bf16", (kvq.KVQ_DECODE_PRIME, 0)),
    "hd64_hpk5_T77_prime_f32": (2, 10, 2, 64, 77, [500, 90], 0, False, "f32", (kvq.KVQ_DECODE_PRIME, 0)),
    "hd128_hpk1_T70_prime_window_f32": (1, 4, 4, 128, 70, [333], 40, True, "f32", (kvq.KVQ_DECODE_PRIME, 0)),
    "hd64_hpk8_T45_prime": (3, 16, 2, 64, 45, [45, 300, 1000], 0, True, "bf16", (kvq.KVQ_DECODE_PRIME, 0)),
    "hd128_T600_prime_window": (1, 8, 2, 128, 600, [2000], 512, False, "bf16", (kvq.KVQ_DECODE_PRIME, 0)),
    "hd64_hpk32_T9_prime_sinks": (2, 32, 1, 64, 9, [200, 9], 0, True, "bf16", None),      # one row per group
    "hd128_hpk3_T41_prime_window_f32": (2, 12, 4, 128, 41, [260, 100], 60, False, "f32", None),   # 30 of 32 rows
}


@pytest.mark.parametrize("name", sorted(MANY))
def test_decode_many_query_rows(name):
    """T * hpk above 32: every query row against the oracle's causal
    attention (row t sees the rows below len - T + t + 1)."""
    B, H, Hkv, hd, T, lens, window, sinks, io, tiling = MANY[name]
    rng = np.random.default_rng(len(name) * 31 + T)
    p = Pair(B, H, Hkv, hd, max(lens) + 8, window, 0, io=io)
    if tiling:
        p.gpu.set_decode_tiling(*tiling)
    k, v = rows(rng, B, max(lens), Hkv, hd, io)
    p.append(k, v, lens)
    q = qrows(rng, B, T, H, hd, io)
    s = rng.standard_normal(H).astype(np.float32) if sinks else None
    p.decode(q, float(np.float32(1 / np.sqrt(hd))), sinks=s, what=name)


IMPORTANCE = {
    # name: (B, H, Hkv, hd, T, lengths, window, cap, step, sinks, io)
    "hd128_gqa": (2, 32, 8, 128, 1, [700, 300], 0, 720, 0, False, "bf16"),
    "hd64_sink_ring": (2, 16, 4, 64, 1, [330, 250], 64, 128, 32, True, "bf16"),
    "hd256_verify_f32": (1, 16, 4, 256, 8, [400], 0, 420, 0, True, "f32"),
    "hd128_prime_window": (1, 8, 2, 128, 40, [300], 100, 320, 0, True, "bf16"),
    # prompt chunks with more (KV head, 16-row tile) pairs than one workgroup
    # per key group takes: 400 and 300 pairs, shared by 13 and 10 workgroups
    "hd128_prime_T200_shared_pairs": (2, 32, 8, 128, 200, [900, 260], 300, 920, 0, True, "bf16"),
    "hd64_prime_T300_shared_pairs_f32": (1, 16, 2, 64, 300, [600], 0, 620, 0, False, "f32"),
}


@pytest.mark.parametrize("name", sorted(IMPORTANCE))
def test_importance_parity(name):
    """Attention importance through the C ABI against the oracle's, after a
    decode of the same query rows supplies the log-sum-exps; a second call
    adds the same mass again."""
    B, H, Hkv, hd, T, lens, window, cap, step, sinks, io = IMPORTANCE[name]
    rng = np.random.default_rng(len(name) + hd)
    p = Pair(B, H, Hkv, hd, cap, window, step, io=io)
    done = np.zeros(B, np.int64)
    while np.any(done < lens):
        n = np.minimum(np.asarray(lens) - done, 32 if step else 400)
        k, v = rows(rng, B, int(n.max()), Hkv, hd, io)
        p.append(k, v, n.tolist())
        done += n
    q = qrows(rng, B, T, H, hd, io)
    s = rng.standard_normal(H).astype(np.float32) if sinks else None
    scale = float(np.float32(1 / np.sqrt(hd)))
    qd = to_dev(q, io)
    sd = torch.from_numpy(s).to(DEV) if s is not None else None
    out, lse = p.gpu.decode(qd, scale, sinks=sd)
    imp = p.gpu.importance(qd, scale, lse)
    torch.cuda.synchronize(DEV)
    want = p.ref.importance(q, scale=scale, sinks=s)
    assert_close(imp.cpu().numpy(), want, name + " importance")
    p.gpu.importance(qd, scale, lse, imp)
    torch.cuda.synchronize(DEV)
    assert_close(imp.cpu().numpy(), 2 * want, name + " importance, second call")
    if s is None:
        np.testing.assert_allclose(imp.sum(1).cpu().numpy(), 2 * T * H, rtol=1e-4)


@pytest.mark.parametrize("fmt", ["q8_0/q5_1", "e4m3"])
def test_registered_importance_follows_rebases(fmt):
    """Importance accumulated step by step in a ring that rebases, with the
    array registered (kvq_set_importance): after every step it holds the
    oracle's mass accumulated per logical row at that row's current physical
    position, and 0 where no live row is stored."""
    rng = np.random.default_rng(31)
    B, H, Hkv, hd, W, step, T = 2, 8, 2, 64, 48, 32, 3
    cap = kvq.kvq_ring_rows(W, T, step)
    p = Pair(B, H, Hkv, hd, cap, W, step, fmt=fmt)
    imp = torch.zeros((B, cap), dtype=torch.float32, device=DEV)
    p.gpu.set_importance(imp)
    acc = [dict() for _ in range(B)]        # logical row -> mass
    scale = float(np.float32(1 / np.sqrt(hd)))
    rebases = 0
    for it in range(70):
        base0 = p.ref.base.copy()
        k, v = rows(rng, B, T, Hkv, hd)
        p.append(k, v)
        rebases += int(np.any(p.ref.base != base0))
        q = qrows(rng, B, T, H, hd)
        qd = to_dev(q, "bf16")
        _, lse = p.gpu.decode(qd, scale)
        p.gpu.importance(qd, scale, lse, imp)
        torch.cuda.synchronize(DEV)
        step_mass = p.ref.importance(q, scale=scale)
        want = np.zeros((B, cap))
        for b in range(B):
            base, ln = int(p.ref.base[b]), int(p.ref.len[b])
            for r in range(ln - base):
                acc[b][base + r] = acc[b].get(base + r, 0.0) + float(step_mass[b][r])
                want[b][r] = acc[b][base + r]
        assert_close(imp.cpu().numpy(), want, f"{fmt} step {it} importance")
    assert rebases >= 3


@pytest.mark.parametrize("step,fmt", [(32, "q8_0/q5_1"), (20, "q8_0/q5_1"), (32, "e4m3"), (64, "e4m3")])
def test_chunked_prime_into_ring(step, fmt):
    """A prompt primed into a sliding-window ring of kvq_ring_rows rows in
    chunks of up to C rows: each chunk's rows are appended, then its rows
    attend causally (each within its window) to what the ring holds, through
    the prime kernel for the 48-row chunks (six groups of query rows) and the
    stream kernel for the smaller ones, whose 32-aligned start stays resident;
    q8_0/q5_1 and FP8 rows.  Every chunk's outputs against the oracle's."""
    rng = np.random.default_rng(21 + step)
    B, H, Hkv, hd, W, C = 2, 16, 4, 64, 64, 48
    cap = kvq.kvq_ring_rows(W, C, step)
    p = Pair(B, H, Hkv, hd, cap, W, step, fmt=fmt)
    s = rng.standard_normal(H).astype(np.float32)
    for it in range(12):
        n = C if it < 8 else int(rng.integers(1, C + 1))
        k, v = rows(rng, B, n, Hkv, hd)
        p.append(k, v)
        p.check_mirror()
        assert np.all((np.maximum(0, p.ref.len - n + 1 - W) & ~31) >= p.ref.base)
        q = qrows(rng, B, n, H, hd)
        p.decode(q, 0.125, sinks=s, what=f"prime chunk {it}")
    assert int(p.ref.base[0]) > 0


@pytest.mark.parametrize("step,tiling", [(24, (kvq.KVQ_DECODE_PER_HEAD, 0)), (32, (kvq.KVQ_DECODE_STREAM, 4)),
                                         (32, (kvq.KVQ_DECODE_STREAM, 0)), (32, (kvq.KVQ_DECODE_AUTO, 0))])
def test_ring_equals_flat(step, tiling):
    """The base-offset ring serves the same rows as a flat cache: identical
    live bytes and identical outputs, step after step, through rebases.  Both
    caches decode with the same kernel (one KV head per workgroup, or the
    kernels that start at a 32-row boundary when the ring's base stays a
    multiple of 32)."""
    rng = np.random.default_rng(11)
    B, H, Hkv, hd, W, cap = 2, 16, 4, 64, 40, 96
    ring = Pair(B, H, Hkv, hd, cap, W, step)
    flat = Pair(B, H, Hkv, hd, 2000, W, 0)
    ring.gpu.set_decode_tiling(*tiling)
    flat.gpu.set_decode_tiling(*tiling)
    L = 0
    for it in range(30):
        n = int(rng.integers(1, 33))
        k, v = rows(rng, B, n, Hkv, hd)
        ring.append(k, v)
        flat.append(k, v)
        L += n
        ring.check_mirror()
        base = int(ring.ref.base[0])
        kr, vr = ring.gpu.planes()
        kf, vf = flat.gpu.planes()
        assert torch.equal(kr[:, :L - base], kf[:, base:L]) and torch.equal(vr[:, :L - base], vf[:, base:L])
        q = qrows(rng, B, 1, H, hd)
        o1, l1 = ring.gpu.decode(to_dev(q, "bf16"), 0.125)
        o2, l2 = flat.gpu.decode(to_dev(q, "bf16"), 0.125)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        if it % 7 == 0:
            ring.decode(q, 0.125, what="ring")
    assert int(ring.ref.base[0]) > 0


def test_truncate_reappend_equals_fresh():
    """Rollback sets len only (memra Cache::rollback): append P+8, truncate to
    P+3, re-append 8 == a fresh cache of the committed P+3 rows plus the 8."""
    rng = np.random.default_rng(12)
    B, H, Hkv, hd, P = 2, 16, 4, 256, 300
    k0, v0 = rows(rng, B, P + 8, Hkv, hd)
    k1, v1 = rows(rng, B, 8, Hkv, hd)
    a = Pair(B, H, Hkv, hd, 400)
    a.append(k0, v0)
    a.truncate([P + 3, P + 3])
    a.check_mirror()
    a.append(k1, v1)
    f = Pair(B, H, Hkv, hd, 400)
    f.append(k0[:, :P + 3], v0[:, :P + 3])
    f.append(k1, v1)
    ka, va = a.gpu.planes()
    kf, vf = f.gpu.planes()
    assert torch.equal(ka[:, :P + 11], kf[:, :P + 11]) and torch.equal(va[:, :P + 11], vf[:, :P + 11])
    q = qrows(rng, B, 8, H, hd)
    oa, la = a.gpu.decode(to_dev(q, "bf16"), 1 / 16)
    of, lf = f.gpu.decode(to_dev(q, "bf16"), 1 / 16)
    assert torch.equal(oa, of) and torch.equal(la, lf)
    a.decode(q, 1 / 16, what="after rollback")


def test_verify_rows_equal_sequential_single_rows():
    """T causal rows == T single-row decodes made as the rows arrive."""
    rng = np.random.default_rng(13)
    B, H, Hkv, hd, N0, T = 2, 16, 4, 128, 500, 8
    k, v = rows(rng, B, N0 + T, Hkv, hd)
    q = qrows(rng, B, T, H, hd)
    a = Pair(B, H, Hkv, hd, 600)
    a.append(k, v)
    oa, la = a.gpu.decode(to_dev(q, "bf16"), 0.088)
    a.decode(q, 0.088, what="T=8")
    s = Pair(B, H, Hkv, hd, 600)
    s.append(k[:, :N0], v[:, :N0])
    for t in range(T):
        s.append(k[:, N0 + t:N0 + t + 1], v[:, N0 + t:N0 + t + 1])
        o1, l1 = s.gpu.decode(to_dev(q[:, t:t + 1], "bf16"), 0.088)
        # equal up to the fp16 rounding of P (Pair.pv_atol)
        np.testing.assert_allclose(o1.cpu().numpy()[:, 0], oa.cpu().numpy()[:, t], atol=a.pv_atol(), rtol=0)
        np.testing.assert_allclose(l1.cpu().numpy()[:, 0], la.cpu().numpy()[:, t], atol=a.lse_atol(), rtol=0)


def test_gqa_equals_repeated_heads():
    rng = np.random.default_rng(14)
    B, H, Hkv, hd, N = 1, 10, 2, 64, 300
    k, v = rows(rng, B, N, Hkv, hd)
    q = qrows(rng, B, 1, H, hd)
    g = Pair(B, H, Hkv, hd, N)
    g.append(k, v)
    r = Pair(B, H, H, hd, N)
    r.append(np.repeat(k, H // Hkv, axis=2), np.repeat(v, H // Hkv, axis=2))
    og, lg = g.gpu.decode(to_dev(q, "bf16"), 0.125)
    orr, lr = r.gpu.decode(to_dev(q, "bf16"), 0.125)
    np.testing.assert_allclose(og.cpu().numpy(), orr.cpu().numpy(), atol=g.pv_atol(), rtol=0)   # fp16 P
    np.testing.assert_allclose(lg.cpu().numpy(), lr.cpu().numpy(), atol=g.lse_atol(), rtol=0)
    g.decode(q, 0.125, what="gqa")


def test_len_one_and_zero_query_closed_forms():
    """len 1: out = V'_0; q = 0: out = mean of the visible V' rows (the oracle
    decodes V'; the GPU must agree within tolerance)."""
    rng = np.random.default_rng(15)
    p = Pair(2, 4, 2, 64, 16, window=5)
    k, v = rows(rng, 2, 1, 2, 64)
    p.append(k, v)
    p.decode(qrows(rng, 2, 1, 4, 64), 0.125, what="len1")
    k, v = rows(rng, 2, 11, 2, 64)
    p.append(k, v)
    p.decode(np.zeros((2, 1, 4, 64), np.float32), 0.125, what="q0")


def test_decode_without_lse_and_f32_inputs():
    rng = np.random.default_rng(16)
    p = Pair(2, 8, 2, 128, 300, io="f32")
    k, v = rows(rng, 2, 250, 2, 128, io="f32")
    p.append(k, v)
    q = qrows(rng, 2, 2, 8, 128, io="f32")
    out, lse = p.gpu.decode(to_dev(q, "f32"), 0.1, want_lse=False)
    assert lse is None
    want, _ = p.ref.attention(q, scale=0.1)
    assert_close(out.cpu().numpy(), want, "f32 no-lse")


def test_host_detected_errors_enqueue_nothing():
    rng = np.random.default_rng(17)
    p = Pair(2, 8, 2, 64, 20)
    k, v = rows(rng, 2, 5, 2, 64)
    p.append(k, v)
    before = [t.clone() for t in p.gpu.planes()]
    with pytest.raises(KvqError) as e:
        p.gpu.decode(to_dev(qrows(rng, 2, 6, 8, 64), "bf16"), 0.1)       # T > len
    assert e.value.status == kvq.KVQ_EINVAL
    with pytest.raises(KvqError) as e:
        p.gpu.append(*(to_dev(x, "bf16") for x in rows(rng, 2, 16, 2, 64)))  # past capacity
    assert e.value.status == kvq.KVQ_ECAPACITY
    with pytest.raises(KvqError):
        p.gpu.truncate([6, 5])
    torch.cuda.synchronize(DEV)
    after = p.gpu.planes()
    assert torch.equal(before[0], after[0]) and torch.equal(before[1], after[1])
    p.check_mirror()
