"""Pin checks of the oracle, each raising AssertionError on a mismatch.

They take the oracle library handle as an argument so that the same checks
can be run against oracle builds with a planted mistake (test_oracle_mutants)
and must fail there.  What fixes each expectation is stated per check; none of
them re-types the oracle's own formula.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
from oracle import core
from oracle.cache_model import OracleCache

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# inputs whose quantization is exact, so the dequantized cache equals them
# ---------------------------------------------------------------------------
def exact_k(rng, n, Hkv, hd):
    """Rows whose q8_0 encoding is exact: each 32-block is c * 2^e with a code
    of magnitude 127 present (then the scale is exactly 2^e)."""
    c = rng.integers(-127, 128, size=(n, Hkv, hd // 32, 32))
    c[..., 0] = 127 * np.where(rng.random((n, Hkv, hd // 32)) < 0.5, 1, -1)
    e = rng.integers(-9, -5, size=(n, Hkv, hd // 32, 1))
    return (c * 2.0 ** e).reshape(n, Hkv, hd).astype(np.float32)


def exact_v(rng, n, Hkv, hd):
    """Rows whose q5_1 encoding is exact: m + c * 2^e, m an fp16 value, codes
    0 and 31 both present."""
    c = rng.integers(0, 32, size=(n, Hkv, hd // 32, 32))
    c[..., 0], c[..., 1] = 0, 31
    e = rng.integers(-6, -3, size=(n, Hkv, hd // 32, 1))
    m = np.float16(1.0) * (rng.standard_normal((n, Hkv, hd // 32, 1)) * 0.5).astype(np.float16)
    return (m.astype(np.float64) + c * 2.0 ** e).reshape(n, Hkv, hd).astype(np.float32)


def exact_f8(rng, n, Hkv, hd):
    """Rows whose FP8 encoding is exact: each 32-block is 2^e times finite
    e4m3 values with one of magnitude 448 (then the scale amax / 448 is
    exactly 2^e and every quotient is its own code)."""
    codes = rng.integers(0, 256, size=(n, Hkv, hd // 32, 32)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C                       # no NaN code
    codes[(codes & 0x7F) == 0x7E] = 0x3D                       # 448 only where placed below
    codes[..., 0] = np.where(rng.random((n, Hkv, hd // 32)) < 0.5, 0x7E, 0xFE)
    e = rng.integers(-10, -3, size=(n, Hkv, hd // 32, 1))
    vals = core.e4m3_value(codes.ravel()).reshape(codes.shape)
    return (vals * 2.0 ** e).reshape(n, Hkv, hd).astype(np.float32)


def sdpa_reference(q, k, v, hpk, scale, window=0, sinks=None):
    """Textbook attention through torch's scaled_dot_product_attention in
    float64 on the CPU.  q [B,T,H,hd]; k, v [B,N,Hkv,hd] (every row, logical
    order).  Query row t of a session of N rows sees rows < N - T + t + 1 (and
    only the last `window` of those); the sink is one extra key with score
    sink_h and value 0."""
    B, T, H, hd = q.shape
    N = k.shape[1]
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)             # B,H,T,hd
    kt = torch.from_numpy(k.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(hpk, 1)
    vt = torch.from_numpy(v.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(hpk, 1)
    j = torch.arange(N)
    upto = N - T + torch.arange(T) + 1
    mask = j[None, :] < upto[:, None]
    if window:
        mask &= j[None, :] >= (upto[:, None] - window)
    if sinks is not None:
        pad = torch.zeros(B, H, T, 1, dtype=torch.float64)
        qt = torch.cat([qt, pad + 1.0], -1)
        kt = torch.cat([kt, torch.zeros(B, H, N, 1, dtype=torch.float64)], -1)
        sk = torch.zeros(B, H, 1, hd + 1, dtype=torch.float64)
        sk[..., hd] = torch.from_numpy(sinks.astype(np.float64))[None, :, None] / scale
        kt = torch.cat([kt, sk], 2)
        vt = torch.cat([vt, torch.zeros(B, H, 1, hd, dtype=torch.float64)], 2)
        mask = torch.cat([mask, torch.ones(T, 1, dtype=torch.bool)], 1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    scores = (qt @ kt.transpose(-1, -2)) * scale
    lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), -1)
    return out.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


def c_append(cache, lib, k, v, counts=None):
    """OracleCache.append, with the codec taken from `lib`."""
    saved = core._lib
    core._lib = lib
    try:
        cache.append(k, v, counts)
    finally:
        core._lib = saved


def attend(cache, lib, q, scale, sinks=None, sel=None):
    saved = core._lib
    core._lib = lib
    try:
        return cache.attention(q, scale=scale, sinks=sinks, sel=sel)
    finally:
        core._lib = saved


# ---------------------------------------------------------------------------
# checks
# ---------------------------------------------------------------------------
def check_golden_codec(lib):
    """Hand-derived block images (tests/golden)."""
    for name, enc, dec, nbytes in (("q8_0_blocks.txt", core.q8_0_encode, core.q8_0_decode, 34),
                                   ("q5_1_blocks.txt", core.q5_1_encode, core.q5_1_decode, 24),
                                   ("f8_blocks.txt", core.f8_encode, core.f8_decode, 34)):
        x = None
        for line in open(os.path.join(GOLDEN, name)):
            line = line.strip()
            if line.startswith("x:"):
                x = np.array([float(t) for t in line[2:].split()], dtype=np.float32)
            elif line.startswith("bytes:"):
                want = np.array([int(t, 16) for t in line[6:].split()], dtype=np.uint8)
                assert np.array_equal(enc(x, lib), want), (name, want)
    # exactly representable records decode to their values
    x = np.array([-2 + 0.25 * i for i in range(32)], np.float32)
    assert np.array_equal(core.q5_1_decode(core.q5_1_encode(x, lib), lib), x.astype(np.float64))
    x = np.array([c * 0.125 for c in range(-16, 16)], np.float32)
    x[0] = -15.875
    assert np.array_equal(core.q8_0_decode(core.q8_0_encode(x, lib), lib), x.astype(np.float64))


def check_f8_rows_golden(lib):
    """FP8 token-row images assembled by hand from the golden blocks
    (tests/golden/f8_rows.txt): the codes of the row's blocks, then their
    scales."""
    blocks = {}
    n = 0
    for line in open(os.path.join(GOLDEN, "f8_blocks.txt")):
        if line.startswith("x:"):
            n += 1
            blocks[n] = np.array([float(t) for t in line[2:].split()], dtype=np.float32)
    seen = 0
    for line in open(os.path.join(GOLDEN, "f8_rows.txt")):
        if line.startswith("blocks:"):
            x = np.concatenate([blocks[int(t)] for t in line[7:].split()])
        elif line.startswith("bytes:"):
            want = np.array([int(t, 16) for t in line[6:].split()], dtype=np.uint8)
            assert np.array_equal(core.quantize_f8_rows(x, x.size, lib), want)
            # the same values as two rows of half the width are two such images
            if x.size == 64:
                two = core.quantize_f8_rows(x, 32, lib).reshape(2, 34)
                for r in range(2):
                    assert np.array_equal(two[r], core.f8_encode(x[32 * r:32 * r + 32], lib)[np.r_[2:34, 0:2]])
            seen += 1
    assert seen == 2


def check_e4m3_codes(lib):
    """Every e4m3 code's value against the format's landmarks (OCP FP8 E4M3:
    largest 448, smallest normal 2^-6, smallest subnormal 2^-9, NaN only at
    S.1111.111, no infinity); the 126 positive finite values rise with the
    code, eight equal steps per binade, and the sign bit only negates."""
    v = core.e4m3_value(np.arange(256), lib)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2
    land = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x40: 2.0,
            0x7E: 448.0, 0x77: 240.0, 0xC0: -2.0, 0xFE: -448.0}
    for c, want in land.items():
        assert v[c] == want, (hex(c), v[c], want)
    assert np.signbit(v[0x80]) and v[0x80] == 0.0
    pos = v[:127]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[128:255], -pos)
    steps = np.diff(pos)
    assert np.all(steps[:8] == 2.0 ** -9)                      # subnormals and the first normal step
    for e in range(1, 15):                                      # binade [2^(e-7), 2^(e-6))
        assert np.all(steps[8 * e: 8 * e + 8] == 2.0 ** (e - 10)), e


def check_e4m3_rounding(lib):
    """Nearest-code rounding against torch's float8_e4m3fn conversion (round
    to nearest even), on every code's value, every midpoint between codes
    (the ties), their float32 neighbours, and log-uniform draws, all within
    +-448 where torch does not turn values into NaN; past 448 the codes
    saturate to +-448."""
    import torch
    pos = core.e4m3_value(np.arange(127), lib)
    mids = (pos[:-1] + pos[1:]) / 2
    m32 = mids.astype(np.float32)
    rng = np.random.default_rng(11)
    draws = np.exp2(rng.uniform(-13, np.log2(448.0), 20000)).astype(np.float32)
    x = np.concatenate([pos.astype(np.float32), m32, np.nextafter(m32, np.float32(0)),
                        np.nextafter(m32, np.float32(np.inf)), draws])
    x = x[np.abs(x) <= 448]
    x = np.concatenate([x, -x])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(core.e4m3_from_f32(x, lib), want)
    big = np.array([448.5, 464, 470, 1e6, 3e38], np.float32)
    assert np.all(core.e4m3_from_f32(big, lib) == 0x7E)
    assert np.all(core.e4m3_from_f32(-big, lib) == 0xFE)


def check_f8_roundtrip(lib):
    """Round trip of FP8 blocks: each value is within half a code step of the
    stored-scale quotient (relative 2^-4 in the normal range, 2^-10 * d among
    the subnormals), plus the stored scale's own shortfall at the saturated
    maximum; a block of codes times an fp16 scale is reproduced exactly."""
    rng = np.random.default_rng(12)
    for dist in ("normal", "outlier", "tiny"):
        x = rng.standard_normal((64, 32)).astype(np.float32)
        if dist == "outlier":
            x[:, 3] *= 40
        if dist == "tiny":
            x *= np.float32(1e-5)
        for blk in x:
            b = core.f8_encode(blk, lib)
            d = float(core.f16_to_f32(b[:2].view(np.uint16), lib)[0])
            y = core.f8_decode(b, lib)
            amax = float(np.abs(blk).max())
            bound = np.maximum(2.0 ** -4 * np.abs(blk), 2.0 ** -10 * d) + max(0.0, amax - 448 * d) + 1e-12
            assert np.all(np.abs(y - blk) <= bound), dist
    codes = rng.integers(0, 256, 32).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10
    codes[0] = 0x7E                                           # the block maximum is 448 * d
    for d in (1.0, 0.25, 2.0 ** -10, 3.0):
        x = (d * core.e4m3_value(codes, lib)).astype(np.float32)
        b = core.f8_encode(x, lib)
        assert np.array_equal(b[2:], np.where(x == 0, codes & 0x80, codes)), d
        assert np.array_equal(core.f8_decode(b, lib), x.astype(np.float64)), d


def check_f16_sample(lib):
    """IEEE binary16 rounding against numpy on a dense sample of every regime."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=400000, dtype=np.uint64).astype(np.uint32)
    e = ((bits >> 23) & 0xFF) % 46 + 100          # exponents 2^-27 .. 2^18
    bits = (bits & 0x807FFFFF) | (e.astype(np.uint32) << 23)
    # plus exact ties at each subnormal and normal quantum
    ties = np.concatenate([(np.arange(1, 2048) + 0.5) * 2.0 ** -24,
                           (1024 + np.arange(0, 1024) + 0.5) * 2.0 ** -10]).astype(np.float32)
    x = np.concatenate([bits.view(np.float32), ties, -ties])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(core.f32_to_f16(x, lib), ref)


def check_textbook(lib, *, B=2, T=3, H=6, Hkv=2, hd=64, N=40, window=0, sinks=False, seed=0, fmt="q8_0/q5_1"):
    """Representable K/V: the oracle must equal textbook attention (torch SDPA,
    float64) over the raw values, with GQA, causal T rows, window and sink;
    for either cache format (values the format stores exactly)."""
    rng = np.random.default_rng(seed)
    if fmt == "e4m3":
        k = exact_f8(rng, B * N, Hkv, hd).reshape(B, N, Hkv, hd)
        v = exact_f8(rng, B * N, Hkv, hd).reshape(B, N, Hkv, hd)
    else:
        k = exact_k(rng, B * N, Hkv, hd).reshape(B, N, Hkv, hd)
        v = exact_v(rng, B * N, Hkv, hd).reshape(B, N, Hkv, hd)
    q = rng.standard_normal((B, T, H, hd)).astype(np.float32)
    s = rng.standard_normal(H).astype(np.float32) if sinks else None
    scale = float(np.float32(1 / np.sqrt(hd)))
    c = OracleCache(B, Hkv, hd, N + 8, window=window, fmt=fmt)
    c_append(c, lib, k, v)
    out, lse = attend(c, lib, q, scale, sinks=s)
    ref, ref_lse = sdpa_reference(q, k, v, H // Hkv, scale, window=window, sinks=s)
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-6, atol=1e-6)


def check_closed_forms(lib, hd=64):
    """len 1: out = V'_0 (no sink) and V'_0 / (1 + e^(sink - s_0)) (sink);
    q = 0: out = mean of the visible rows of V'."""
    rng = np.random.default_rng(3)
    k = exact_k(rng, 1, 1, hd).reshape(1, 1, 1, hd)
    v = exact_v(rng, 1, 1, hd).reshape(1, 1, 1, hd)
    q = rng.standard_normal((1, 1, 2, hd)).astype(np.float32)
    scale = 0.125
    c = OracleCache(1, 1, hd, 4)
    c_append(c, lib, k, v)
    out, lse = attend(c, lib, q, scale)
    assert np.array_equal(out[0, 0, 0], v[0, 0, 0]) and np.array_equal(out[0, 0, 1], v[0, 0, 0])
    s0 = scale * (q[0, 0].astype(np.float64) @ k[0, 0, 0].astype(np.float64))
    np.testing.assert_allclose(lse[0, 0], s0, rtol=1e-6, atol=1e-6)
    sink = np.array([0.7, -1.3], np.float32)
    out, _ = attend(c, lib, q, scale, sinks=sink)
    for h in range(2):
        want = v[0, 0, 0].astype(np.float64) / (1 + np.exp(float(sink[h]) - s0[h]))
        np.testing.assert_allclose(out[0, 0, h], want, rtol=1e-6, atol=1e-7)
    # q = 0 with a window of 5 over 12 rows: mean of the last 5 rows
    N, W = 12, 5
    k = exact_k(rng, N, 1, hd).reshape(1, N, 1, hd)
    v = exact_v(rng, N, 1, hd).reshape(1, N, 1, hd)
    c = OracleCache(1, 1, hd, N, window=W)
    c_append(c, lib, k, v)
    out, _ = attend(c, lib, np.zeros((1, 1, 1, hd), np.float32), scale)
    np.testing.assert_allclose(out[0, 0, 0], v[0, N - W:, 0].astype(np.float64).mean(0), rtol=1e-6, atol=1e-7)


def check_causal_rows_equal_sequential(lib):
    """A T-row call equals T single-row calls made as the rows arrive
    (cortiq attend_group_upto: bit-identical to append-then-attend)."""
    rng = np.random.default_rng(5)
    B, H, Hkv, hd, N0, T = 2, 4, 2, 64, 20, 6
    k = rng.standard_normal((B, N0 + T, Hkv, hd)).astype(np.float32)
    v = rng.standard_normal((B, N0 + T, Hkv, hd)).astype(np.float32)
    q = rng.standard_normal((B, T, H, hd)).astype(np.float32)
    for window in (0, 7):
        a = OracleCache(B, Hkv, hd, 64, window=window)
        c_append(a, lib, k, v)
        out, lse = attend(a, lib, q, 0.125)
        s = OracleCache(B, Hkv, hd, 64, window=window)
        c_append(s, lib, k[:, :N0], v[:, :N0])
        for t in range(T):
            c_append(s, lib, k[:, N0 + t:N0 + t + 1], v[:, N0 + t:N0 + t + 1])
            o1, l1 = attend(s, lib, q[:, t:t + 1], 0.125)
            assert np.array_equal(o1[:, 0], out[:, t]) and np.array_equal(l1[:, 0], lse[:, t])


def check_gqa_equals_repeated_heads(lib):
    """Grouped attention equals per-head attention over KV heads repeated hpk
    times (cortiq attend_group: identical per head)."""
    rng = np.random.default_rng(6)
    B, H, Hkv, hd, N = 1, 6, 2, 64, 30
    k = rng.standard_normal((B, N, Hkv, hd)).astype(np.float32)
    v = rng.standard_normal((B, N, Hkv, hd)).astype(np.float32)
    q = rng.standard_normal((B, 1, H, hd)).astype(np.float32)
    g = OracleCache(B, Hkv, hd, N)
    c_append(g, lib, k, v)
    out, lse = attend(g, lib, q, 0.125)
    r = OracleCache(B, H, hd, N)
    c_append(r, lib, np.repeat(k, H // Hkv, axis=2), np.repeat(v, H // Hkv, axis=2))
    o2, l2 = attend(r, lib, q, 0.125)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)


def check_ring_equals_flat(lib):
    """A windowed ring (physical row = row - base) serves the same bytes and the
    same attention as a flat cache with the same window."""
    rng = np.random.default_rng(8)
    B, H, Hkv, hd, W, cap, step = 2, 4, 2, 32, 8, 16, 4
    flat = OracleCache(B, Hkv, hd, 200, window=W)
    ring = OracleCache(B, Hkv, hd, cap, window=W, ring_step=step)
    L = 0
    for n in [3, 1, 5, 1, 1, 2, 6, 1, 4, 6, 1, 1, 6, 2, 1, 5, 3, 1, 1, 1, 1, 4]:
        k = rng.standard_normal((B, n, Hkv, hd)).astype(np.float32)
        v = rng.standard_normal((B, n, Hkv, hd)).astype(np.float32)
        c_append(flat, lib, k, v)
        c_append(ring, lib, k, v)
        L += n
        base = int(ring.base[0])
        assert L - base <= cap and (base == 0 or max(0, L - n + 1 - W) >= base)
        for b in range(B):
            assert np.array_equal(ring.k[b, :L - base], flat.k[b, base:L])
            assert np.array_equal(ring.v[b, :L - base], flat.v[b, base:L])
        q = rng.standard_normal((B, 1, H, hd)).astype(np.float32)
        o1, l1 = attend(flat, lib, q, 0.17)
        assert np.array_equal(ring.len, flat.len)
        o2, l2 = attend(ring, lib, q, 0.17)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def check_truncate_equals_fresh(lib):
    """Rollback = set len (memra Cache::rollback): append P+8, truncate to P+3,
    re-append 8 equals a fresh cache given the committed P+3 rows and the same 8."""
    rng = np.random.default_rng(9)
    B, H, Hkv, hd, P = 2, 8, 2, 64, 25
    rows = rng.standard_normal((B, P + 16, Hkv, hd)).astype(np.float32)
    vals = rng.standard_normal((B, P + 16, Hkv, hd)).astype(np.float32)
    a = OracleCache(B, Hkv, hd, 64)
    c_append(a, lib, rows[:, :P + 8], vals[:, :P + 8])
    a.truncate(np.full(B, P + 3))
    new_k = rng.standard_normal((B, 8, Hkv, hd)).astype(np.float32)
    new_v = rng.standard_normal((B, 8, Hkv, hd)).astype(np.float32)
    c_append(a, lib, new_k, new_v)
    f = OracleCache(B, Hkv, hd, 64)
    c_append(f, lib, rows[:, :P + 3], vals[:, :P + 3])
    c_append(f, lib, new_k, new_v)
    assert np.array_equal(a.k[:, :P + 11], f.k[:, :P + 11]) and np.array_equal(a.v[:, :P + 11], f.v[:, :P + 11])
    q = rng.standard_normal((B, 8, H, hd)).astype(np.float32)
    o1, l1 = attend(a, lib, q, 0.125)
    o2, l2 = attend(f, lib, q, 0.125)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def importance_of(cache, lib, q, scale, sinks=None):
    saved = core._lib
    core._lib = lib
    try:
        return cache.importance(q, scale=scale, sinks=sinks)
    finally:
        core._lib = saved


def check_importance_textbook(lib, *, B=2, T=3, H=6, Hkv=2, hd=64, N=40, window=9, sinks=True, seed=3,
                              fmt="q8_0/q5_1"):
    """Representable K: the importance equals a textbook softmax (torch,
    float64) of every (query row, head) over its visible rows plus the sink as
    one more column, the row columns summed over heads and query rows; rows
    that no query row sees, and physical rows past len, hold 0."""
    rng = np.random.default_rng(seed)
    k = (exact_f8 if fmt == "e4m3" else exact_k)(rng, B * N, Hkv, hd).reshape(B, N, Hkv, hd)
    v = np.zeros_like(k)
    q = rng.standard_normal((B, T, H, hd)).astype(np.float32)
    s = rng.standard_normal(H).astype(np.float32) if sinks else None
    scale = float(np.float32(1 / np.sqrt(hd)))
    c = OracleCache(B, Hkv, hd, N + 8, window=window, fmt=fmt)
    c_append(c, lib, k, v)
    imp = importance_of(c, lib, q, scale, sinks=s)
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)                       # B,H,T,hd
    kt = torch.from_numpy(k.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(H // Hkv, 1)
    scores = (qt @ kt.transpose(-1, -2)) * scale                                          # B,H,T,N
    j = torch.arange(N)
    upto = N - T + torch.arange(T) + 1
    mask = j[None, :] < upto[:, None]
    if window:
        mask &= j[None, :] >= (upto[:, None] - window)
    scores = scores.masked_fill(~mask, float("-inf"))
    if s is not None:
        col = torch.from_numpy(s.astype(np.float64))[None, :, None, None].expand(B, H, T, 1)
        scores = torch.cat([scores, col], -1)
    p = torch.softmax(scores, -1)[..., :N]
    want = np.zeros((B, N + 8))
    want[:, :N] = p.sum(dim=(1, 2)).numpy()
    np.testing.assert_allclose(imp, want, rtol=1e-10, atol=1e-13)


def check_importance_mass(lib):
    """Without sinks every (query row, head) spreads probability 1 over its
    rows: the importance of a session sums to T * H."""
    rng = np.random.default_rng(4)
    B, T, H, Hkv, hd, N = 3, 5, 8, 2, 32, 50
    c = OracleCache(B, Hkv, hd, N, window=17)
    k = (rng.standard_normal((B, N, Hkv, hd)) * 3).astype(np.float32)
    c_append(c, lib, k, k, [N, N - 7, T])
    imp = importance_of(c, lib, rng.standard_normal((B, T, H, hd)).astype(np.float32), 0.2)
    np.testing.assert_allclose(imp.sum(1), T * H, rtol=1e-12)
    assert np.all(imp >= 0)


ALL_CHECKS = {
    "golden_codec": check_golden_codec,
    "f8_rows_golden": check_f8_rows_golden,
    "textbook_f8": lambda lib: check_textbook(lib, B=2, T=3, H=8, Hkv=4, hd=64, N=37, window=11, sinks=True,
                                              seed=21, fmt="e4m3"),
    "textbook_f8_hd256": lambda lib: check_textbook(lib, B=1, T=8, H=8, Hkv=2, hd=256, N=29, seed=22, fmt="e4m3"),
    "importance_textbook_f8": lambda lib: check_importance_textbook(lib, B=1, T=2, H=8, Hkv=4, hd=96, N=30,
                                                                     window=0, sinks=True, seed=23, fmt="e4m3"),
    "f16_sample": check_f16_sample,
    "e4m3_codes": check_e4m3_codes,
    "e4m3_rounding": check_e4m3_rounding,
    "f8_roundtrip": check_f8_roundtrip,
    "textbook": check_textbook,
    "textbook_window_sink": lambda lib: check_textbook(lib, window=9, sinks=True, T=4, seed=1),
    "textbook_hd128": lambda lib: check_textbook(lib, B=1, T=1, H=8, Hkv=8, hd=128, N=33, seed=2),
    "closed_forms": check_closed_forms,
    "causal_rows": check_causal_rows_equal_sequential,
    "gqa_repeat": check_gqa_equals_repeated_heads,
    "ring_flat": check_ring_equals_flat,
    "truncate_fresh": check_truncate_equals_fresh,
    "importance_textbook": check_importance_textbook,
    "importance_textbook_gqa4": lambda lib: check_importance_textbook(lib, B=1, T=2, H=8, Hkv=2, hd=96,
                                                                       N=30, window=0, sinks=False, seed=5),
    "importance_mass": check_importance_mass,
}
