"""GPU parity of the FP8 (e4m3) K/V variant (memra-engine "Module cache"
page, kv_fp8_on) through the C ABI against the oracle: FP8 rows (the codes of
a row's blocks, then their fp16 scales) byte for byte after every append, and
decode outputs and log-sum-exps within |gpu - oracle| <= 2e-3 + 1e-2 |oracle|
(2e-3 relative to the V scale for large V, as in test_gpu_range) on the
layouts the stream kernel has and on prompt chunks (the prime kernel),
every e4m3 code read back, attention importance, and the large-V, large- and
tiny-K and extreme-query range.
"""
import numpy as np
import pytest
import torch

from decode_attention_quantized_append_amd import kvq
from decode_attention_quantized_append_amd.workloads import round_bf16

pytestmark = pytest.mark.gpu

from gpu_pair import ATOL, DEV, Pair, assert_close, to_dev  # noqa: E402

F8 = "e4m3"


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


# -- append: FP8 rows bit-exact ------------------------------------------------------
@pytest.mark.parametrize("B,Hkv,hd,io", [(1, 1, 64, "f32"), (2, 8, 128, "bf16"), (3, 4, 256, "bf16"),
                                         (2, 2, 64, "bf16"), (1, 3, 128, "f32")])
def test_f8_append_rows_bit_exact(B, Hkv, hd, io):
    rng = np.random.default_rng(hd * 11 + B + Hkv)
    p = Pair(B, 4 * Hkv, Hkv, hd, 400, io=io, fmt=F8)
    for T, counts in [(1, None), (7, None), (64, [64 - b for b in range(B)]), (130, None), (3, [0] + [3] * (B - 1))]:
        k, v = rows(rng, B, T, Hkv, hd, io, scale=rng.choice([1e-4, 1.0, 300.0]), outliers=(hd == 128))
        p.append(k, v, counts)
        p.check_mirror()
    p.check_planes()


def test_f8_append_edge_blocks():
    """Ties between e4m3 neighbours at a scale of 1 (amax 448), the subnormal
    range, saturation (an fp16 scale below amax/448), signed zeros, zero
    blocks, one-hot blocks and ranges from 1e-6 to 6e4: every byte equals
    the oracle's, for K and for V."""
    hd = 32 * 8
    blocks = []
    tie = np.zeros(32, np.float32)
    tie[0] = 448.0
    tie[1:16] = [1.0625, 1.1875, 17, 19, 100, 14.5, 0.5 * 2.0 ** -9, 1.5 * 2.0 ** -9, 7.5 * 2.0 ** -9,
                 -2.0 ** -10, 3.5 * 2.0 ** -9, 240 + 8, 464 * 0.96, 1.9375, 2.0 ** -6]
    tie[16:] = -tie[1:17]
    blocks.append(tie)
    sat = np.full(32, 0.03, np.float32)
    sat[0], sat[1], sat[2] = 1.0, -1.0, 16.998 / 448
    blocks.append(sat)
    blocks.append(np.zeros(32, np.float32))
    blocks.append(np.full(32, -0.0, np.float32))
    one = np.zeros(32, np.float32)
    one[9] = -5.0
    one[10] = -0.0
    blocks.append(one)
    blocks.append(np.linspace(-6e4, 6e4, 32).astype(np.float32))
    blocks.append((np.arange(32) * 1e-7).astype(np.float32))
    rng = np.random.default_rng(4)
    blocks.append((rng.standard_normal(32) * 10.0 ** rng.integers(-5, 4)).astype(np.float32))
    row = np.concatenate(blocks).reshape(1, 1, 2, hd // 2)
    for io in ("f32", "bf16"):
        x = row if io == "f32" else round_bf16(row)
        p = Pair(1, 2, 2, hd // 2, 4, io=io, fmt=F8)
        p.append(x, -x)
        p.append(x[:, :, :, ::-1].copy(), x)
        p.check_planes()


# -- decode parity -----------------------------------------------------------------
SHAPES = {
    # name: (B, H, Hkv, hd, T, lengths, window, cap, step, sinks, io, outliers, tiling)
    "tiny": (1, 4, 1, 64, 1, [256], 0, 300, 0, False, "f32", False, None),
    "qwen_gqa": (1, 32, 8, 128, 1, [1500], 0, 1600, 0, False, "bf16", True, None),
    "batched_ragged": (16, 40, 8, 128, 1, [1, 2, 63, 64, 65, 127, 128, 129, 700, 1023, 1024, 1025,
                                           333, 900, 5, 1100], 0, 1200, 0, False, "bf16", False, None),
    "batched_long_rowstreams": (2, 40, 8, 128, 1, [3000, 2100], 0, 3100, 0, False, "bf16", False, None),
    "sink_ring": (4, 64, 8, 64, 1, [1000, 1000, 1000, 1000], 64, 128, 32, True, "bf16", False, None),
    "verify_dimhalves": (2, 16, 4, 256, 8, [600, 333], 0, 700, 0, False, "bf16", False, None),
    "verify_f32_sinks": (2, 16, 4, 256, 8, [500, 75], 0, 600, 0, True, "f32", False, None),
    "hd128_T8_dimhalves": (2, 16, 4, 128, 8, [420, 97], 50, 450, 0, True, "bf16", False, None),
    "hd64_rowgroups": (2, 24, 1, 64, 1, [400, 77], 0, 420, 0, False, "bf16", False, (kvq.KVQ_DECODE_STREAM, 0, 2)),
    "hd256_rowtiles": (1, 16, 4, 256, 8, [300], 0, 320, 0, False, "bf16", False, (kvq.KVQ_DECODE_STREAM, 0, 1)),
    "hd128_headgroup2": (2, 32, 8, 128, 2, [900, 161], 0, 1000, 0, True, "f32", True, (kvq.KVQ_DECODE_STREAM, 2, 0)),
    "prime_T100": (1, 32, 8, 128, 100, [700], 300, 720, 0, True, "bf16", True, None),
    # more prompt chunks on the prime kernel: head_dim 64 with fp32 inputs, a
    # sliding-window ring, one query row per group (32 query heads per KV
    # head), 30 of 32 rows per group (3 query heads per KV head)
    "prime_hd64_f32": (2, 16, 4, 64, 40, [500, 90], 0, 560, 0, False, "f32", False, (kvq.KVQ_DECODE_PRIME, 0, 0)),
    "prime_ring": (2, 8, 2, 64, 40, [600, 300], 200, 400, 32, False, "f32", False, (kvq.KVQ_DECODE_PRIME, 0, 0)),
    "prime_hpk32_sinks": (2, 32, 1, 64, 9, [200, 9], 0, 220, 0, True, "bf16", False, None),
    "prime_hd128_hpk3_window": (2, 12, 4, 128, 41, [260, 100], 60, 280, 0, False, "f32", True, None),
}


def build(name, seed=0, v_scale=1.0, k_scale=1.0):
    B, H, Hkv, hd, T, lens, window, cap, step, sinks, io, outl, tiling = SHAPES[name]
    rng = np.random.default_rng(seed + 17 * len(name))
    p = Pair(B, H, Hkv, hd, cap, window, step, io=io, fmt=F8)
    if tiling:
        p.gpu.set_decode_tiling(*tiling)
    lens = np.asarray(lens)
    done = np.zeros(B, np.int64)
    piece = 32 if step else 400
    while np.any(done < lens):
        n = np.minimum(lens - done, piece)
        k, v = rows(rng, B, int(n.max()), Hkv, hd, io, outliers=outl)
        if v_scale != 1.0:
            v = v * np.float32(v_scale)
            v = round_bf16(v) if io == "bf16" else v
        if k_scale != 1.0:
            k = k * np.float32(k_scale)
            k = round_bf16(k) if io == "bf16" else k
        p.append(k, v, n.tolist())
        done += n
    q = qrows(rng, B, T, H, hd, io)
    if k_scale != 1.0:
        q = q * np.float32(1.0 / k_scale)
        q = round_bf16(q) if io == "bf16" else q
    s = rng.standard_normal(H).astype(np.float32) if sinks else None
    return p, q, s, float(np.float32(1 / np.sqrt(hd)))


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_f8_decode_parity(name):
    p, q, s, scale = build(name)
    p.check_planes()
    print(f"\ncase {name}", flush=True)
    p.decode(q, scale, sinks=s, what=f"f8 {name}")


@pytest.mark.parametrize("name", ["verify_dimhalves", "qwen_gqa", "hd64_rowgroups", "prime_T100", "prime_hd64_f32"])
def test_f8_decode_large_v(name):
    """V blocks of range up to 3e5 (steps to about 700, scale shift on)."""
    p, q, s, scale = build(name, seed=3, v_scale=1e5)
    atol = ATOL * max(1.0, 1.05 * p.vmax / 4.0)
    p.decode(q, scale, sinks=s, what=f"f8 {name} large v", atol=atol)


@pytest.mark.parametrize("k_scale", [3e4, 1e-5])
@pytest.mark.parametrize("name", ["qwen_gqa", "verify_dimhalves", "prime_T100", "prime_hd64_f32"])
def test_f8_decode_large_and_tiny_k(name, k_scale):
    """K rows times 3e4 (block scales of about 2^8, past the prime kernel's
    K shift at 2^7) or times 1e-5 (subnormal fp16 scales), with the queries
    divided by the same factor so that the scores keep their size."""
    p, q, s, scale = build(name, seed=5, k_scale=k_scale)
    print(f"\ncase {name} k x{k_scale:g}", flush=True)
    p.decode(q, scale, sinks=s, what=f"f8 {name} k x{k_scale:g}")


@pytest.mark.parametrize("name", ["qwen_gqa", "verify_f32_sinks", "prime_T100", "prime_hd64_f32"])
def test_f8_decode_extreme_queries(name):
    """Query rows of magnitudes 1e5, 1e-6, 1e-30, 0 and single spikes mixed
    within every group of rows (the classes of test_gpu_range)."""
    from test_gpu_range import extreme_q
    p, _, s, scale = build(name, seed=7)
    B, H, Hkv, hd, T, *_ = SHAPES[name]
    q = extreme_q(np.random.default_rng(11), B, T, H, hd, SHAPES[name][10])
    print(f"\ncase {name} extreme q", flush=True)
    p.decode(q, scale, sinks=s, what=f"f8 {name} extreme q")


def test_f8_decode_every_code():
    """Rows written directly with every finite e4m3 code (the two NaN codes
    replaced): at length 1 the output is V'_0 exactly (one visible row,
    weight 1) and the lse is the scaled score of that row, so every code's
    value is read back through both the K and the V path; then a second row
    and a query of zeros give the mean of the two V rows."""
    hd, Hkv = 256, 1
    p = Pair(1, 2, Hkv, hd, 8, io="f32", fmt=F8)
    z = np.zeros((1, 2, Hkv, hd), np.float32)
    p.append(z, z)
    codes = np.arange(256, dtype=np.uint8)
    codes[0x7F], codes[0xFF] = 0x3B, 0xBB
    scales = np.array([0x3C00, 0x3800, 0x4000, 0x2C00, 0x5000, 0x3C00, 0x1800, 0x4400], np.uint16)
    row0 = np.concatenate([codes, scales.view(np.uint8)])
    row1 = np.concatenate([codes[::-1].copy(), scales[::-1].copy().view(np.uint8)])
    kp, vp = p.gpu.planes()
    for r, img in enumerate((row0, row1)):
        t = torch.from_numpy(img).to(DEV)
        kp[0, r].copy_(t)
        vp[0, r].copy_(t)
        p.ref.k[0, r] = img
        p.ref.v[0, r] = img
    p.check_planes()
    rng = np.random.default_rng(9)
    p.truncate([1])
    q = rng.standard_normal((1, 1, 2, hd)).astype(np.float32)
    got = p.decode(q, 0.0625, what="f8 every code, len 1")
    want, _ = p.ref.attention(q, scale=0.0625)
    out, _ = p.gpu.decode(to_dev(q, "f32"), 0.0625)
    torch.cuda.synchronize(DEV)
    assert np.array_equal(out.cpu().numpy(), want), "len 1: out must be V'_0 exactly"
    assert got == 0.0
    p.ref.len[:] = 2
    p.gpu.set_host_lengths([2], [0])
    p.gpu.counters[0] = 2
    p.decode(np.zeros((1, 1, 2, hd), np.float32), 0.0625, what="f8 every code, mean of two rows")


def test_f8_importance_parity():
    rng = np.random.default_rng(31)
    for B, H, Hkv, hd, T, lens, window, cap, step, sinks, io in (
            (2, 32, 8, 128, 1, [700, 300], 0, 720, 0, False, "bf16"),
            (2, 16, 4, 64, 1, [330, 250], 64, 128, 32, True, "bf16"),
            (1, 16, 4, 256, 8, [400], 0, 420, 0, True, "f32"),
            (1, 32, 8, 128, 160, [700], 0, 720, 0, False, "bf16")):   # 320 pairs, 10 workgroups per key group
        p = Pair(B, H, Hkv, hd, cap, window, step, io=io, fmt=F8)
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
        assert_close(imp.cpu().numpy(), want, f"f8 importance hd{hd}")


def test_f8_ring_equals_flat():
    """An FP8 ring serves the same rows as a flat FP8 cache: identical live
    bytes and outputs through rebases."""
    rng = np.random.default_rng(13)
    B, H, Hkv, hd, W, cap, step = 2, 16, 4, 64, 40, 96, 32
    ring = Pair(B, H, Hkv, hd, cap, W, step, fmt=F8)
    flat = Pair(B, H, Hkv, hd, 2000, W, 0, fmt=F8)
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
            ring.decode(q, 0.125, what="f8 ring")
    assert int(ring.ref.base[0]) > 0


def test_f8_per_head_kernel_is_refused():
    p, q, s, scale = build("qwen_gqa")
    p.gpu.set_decode_tiling(kvq.KVQ_DECODE_PER_HEAD, 0, 0)
    with pytest.raises(kvq.KvqError) as e:
        p.gpu.decode(to_dev(q, "bf16"), scale)
    assert e.value.status == kvq.KVQ_EINVAL


# Kernels and tilings (kernel, KV heads per workgroup, waves per KV head) that
# fit each FP8 shape: the prime kernel and the stream kernel's layouts.
PR, ST, AUTO = kvq.KVQ_DECODE_PRIME, kvq.KVQ_DECODE_STREAM, kvq.KVQ_DECODE_AUTO
F8_TILINGS = {
    "qwen_gqa": [(ST, 8, 0), (ST, 4, 0), (ST, 2, 0), (ST, 8, 1), (ST, 8, 2)],
    "verify_dimhalves": [(ST, 0, 0), (ST, 1, 3), (ST, 2, 3), (ST, 4, 3), (ST, 0, 2), (ST, 0, 1)],
    "hd128_T8_dimhalves": [(ST, 1, 3), (ST, 2, 3), (ST, 0, 2)],
    "prime_T100": [(PR, 0, 0), (ST, 0, 0), (ST, 0, 3), (ST, 0, 2)],
    "prime_hd64_f32": [(PR, 0, 0), (ST, 0, 0), (ST, 0, 2)],
}


@pytest.mark.parametrize("name", sorted(F8_TILINGS))
def test_f8_plans_exact_weights(name):
    """With zero queries every visible row scores 0 and every weight is
    exactly 1, and so is each weight times its FP8 step: the output is the
    mean of the visible V rows (the sink in the denominator) up to the fp32
    summation, for every kernel, tiling and split plan, within 1e-5 of the V
    scale (a row dropped, counted twice or masked wrongly shows up)."""
    p, q, s, scale = build(name)
    q = np.zeros_like(q)
    io = SHAPES[name][10]
    qd = to_dev(q, io)
    sd = torch.from_numpy(s).to(DEV) if s is not None else None
    want, want_lse = p.ref.attention(q, scale=scale, sinks=s)
    atol = 1e-5 * max(1.0, p.vmax)
    for kernel, gh, sub in [(AUTO, 0, 0)] + F8_TILINGS[name]:
        p.gpu.set_decode_tiling(kernel, gh, sub)
        for rows_ in (0, 64, 256):
            p.gpu.set_split_rows(rows_)
            o, l = p.gpu.decode(qd, scale, sinks=sd)
            what = f"f8 {name} kernel={kernel} gh={gh} sub={sub} split={rows_}"
            np.testing.assert_allclose(o.cpu().numpy(), want, atol=atol, rtol=0, err_msg=what)
            np.testing.assert_allclose(l.cpu().numpy(), want_lse, atol=1e-5, rtol=0, err_msg=what)
