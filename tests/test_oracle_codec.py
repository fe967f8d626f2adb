"""Pins of the oracle's codec (CPU only).

What fixes each expectation:
* byte sizes 34 / 24 per 32 elements -- memra-engine "Struct KvLayer" page;
* block images in tests/golden -- derived by hand from the format reading;
* fp16 rounding -- IEEE 754, checked against numpy's float16 conversion;
* round-trip bound |x - x'| <= d/2 (q8_0) and <= d/2 + |min - stored min|
  (q5_1), d the stored scale -- the rounding of a code is at most half a step;
* exact reproduction of blocks whose values are representable;
* half-to-even on constructed ties.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _records(name):
    recs, x = [], None
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line.startswith("x:"):
            x = np.array([float(v) for v in line[2:].split()], dtype=np.float32)
        elif line.startswith("bytes:"):
            recs.append((x, np.array([int(v, 16) for v in line[6:].split()], dtype=np.uint8)))
    return recs


# -- fp16 conversion ------------------------------------------------------
def test_f16_matches_numpy_on_every_float_in_range():
    """Every float32 whose exponent lies in [2^-27, 2^17): all 2^23 significands
    for each exponent and both signs, i.e. every rounding case of binary16
    (normal, subnormal, underflow to 0, overflow to inf)."""
    lib = oracle.load()
    mant = np.arange(1 << 23, dtype=np.uint32)
    for e in range(127 - 27, 127 + 17):
        for s in (0, 1):
            bits = (np.uint32(s) << 31) | (np.uint32(e) << 23) | mant
            x = bits.view(np.float32)
            with np.errstate(over="ignore"):
                ref = x.astype(np.float16).view(np.uint16)
            got = oracle.f32_to_f16(x, lib)
            bad = np.nonzero(got != ref)[0]
            assert bad.size == 0, (e, s, hex(int(bits[bad[0]])), hex(int(got[bad[0]])), hex(int(ref[bad[0]])))


def test_f16_special_values():
    x = np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.99, 65520.0, 1e-30,
                  2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14], dtype=np.float32)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f32_to_f16(x), ref)
    nan = oracle.f32_to_f16(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0


def test_f16_to_f32_is_exact_widening():
    h = np.arange(1 << 16, dtype=np.uint16)
    finite = (h & 0x7C00) != 0x7C00
    got = oracle.f16_to_f32(h[finite])
    assert np.array_equal(got, h[finite].view(np.float16).astype(np.float32))


# -- golden block images ----------------------------------------------------
@pytest.mark.parametrize("i", range(5))
def test_q8_0_golden(i):
    x, want = _records("q8_0_blocks.txt")[i]
    assert x.size == 32 and want.size == 34
    assert np.array_equal(oracle.q8_0_encode(x), want)
    # decode of the golden bytes: d * code, compared with the hand values where exact
    d16 = int(want[0]) | (int(want[1]) << 8)
    d = float(np.array([d16], np.uint16).view(np.float16)[0])
    codes = want[2:].view(np.int8).astype(np.float64)
    assert np.array_equal(oracle.q8_0_decode(want), d * codes)


@pytest.mark.parametrize("i", range(5))
def test_q5_1_golden(i):
    x, want = _records("q5_1_blocks.txt")[i]
    assert x.size == 32 and want.size == 24
    assert np.array_equal(oracle.q5_1_encode(x), want)


def test_q5_1_golden_decodes_to_hand_values():
    # records 1-3 are exactly representable: decoding gives x back
    for x, blk in _records("q5_1_blocks.txt")[:3]:
        assert np.array_equal(oracle.q5_1_decode(blk), x.astype(np.float64))


def test_block_sizes_match_the_pages():
    x = np.random.default_rng(0).standard_normal(32).astype(np.float32)
    assert oracle.q8_0_encode(x).size == 34
    assert oracle.q5_1_encode(x).size == 24
    assert oracle.quantize_k(np.zeros(128, np.float32)).size == 4 * 34
    assert oracle.quantize_v(np.zeros(128, np.float32)).size == 4 * 24


# -- exact reproduction of representable blocks ------------------------------
@pytest.mark.parametrize("e", [-20, -8, -3, 0, 4, 9])
def test_q8_0_exact_blocks(e):
    rng = np.random.default_rng(e + 100)
    c = rng.integers(-127, 128, size=32)
    c[rng.integers(32)] = 127 * (1 if rng.random() < 0.5 else -1)
    x = (c * 2.0 ** e).astype(np.float32)
    blk = oracle.q8_0_encode(x)
    assert np.array_equal(blk[2:].view(np.int8), c.astype(np.int8))
    assert np.array_equal(oracle.q8_0_decode(blk), x.astype(np.float64))


@pytest.mark.parametrize("e", [-10, -4, -2, 0, 3])
def test_q5_1_exact_blocks(e):
    rng = np.random.default_rng(e + 200)
    c = rng.permutation(np.concatenate([[0, 31], rng.integers(0, 32, size=30)]))
    mn = float(np.float16(rng.standard_normal() * 4))         # an fp16 offset
    x = (mn + c * 2.0 ** e).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), mn + c * 2.0 ** e)  # representable
    got = oracle.q5_1_decode(oracle.q5_1_encode(x))
    assert np.array_equal(got, x.astype(np.float64))


def test_q8_0_ties_round_half_even():
    d = 2.0 ** -3
    k = np.arange(-20, 20)
    x = np.zeros(32, np.float32)
    x[0] = 127 * d
    for start in range(0, 40, 31):
        ks = k[start:start + 31]
        x[1:1 + ks.size] = (ks + 0.5) * d
        blk = oracle.q8_0_encode(x)
        got = blk[3:3 + ks.size].view(np.int8)
        assert np.array_equal(got, np.round(ks + 0.5).astype(np.int8))  # numpy rounds half to even


def test_q5_1_ties_round_half_even():
    x = np.zeros(32, np.float32)
    x[0], x[1] = 0.0, 31 * 0.25
    k = np.arange(0, 30)
    x[2:] = (k + 0.5) * 0.25
    blk = oracle.q5_1_encode(x)
    codes = _unpack_q5_1(blk)
    assert np.array_equal(codes[2:], np.round(k + 0.5))


def _unpack_q5_1(blk):
    qh = int.from_bytes(bytes(blk[4:8]), "little")
    nib = blk[8:24]
    lo = nib & 15
    hi = nib >> 4
    c = np.concatenate([lo, hi]).astype(np.int64)
    return c | (((qh >> np.arange(32)) & 1) << 4)


# -- round-trip error bounds ---------------------------------------------------
def _normal_blocks(n, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal((n, 32)) * scale).astype(np.float32)


@pytest.mark.parametrize("scale", [0.05, 1.0, 37.0])
def test_q8_0_roundtrip_bound(scale):
    x = _normal_blocks(4000, 1, scale)
    blk = oracle.quantize_k(x).reshape(-1, 34)
    for i in range(x.shape[0]):
        d = float(blk[i, :2].view(np.float16)[0])
        xr = oracle.q8_0_decode(blk[i])
        assert np.all(np.abs(x[i] - xr) <= d / 2 * (1 + 2.0 ** -16)), i


@pytest.mark.parametrize("scale", [0.05, 1.0, 37.0])
def test_q5_1_roundtrip_bound(scale):
    x = _normal_blocks(4000, 2, scale)
    blk = oracle.quantize_v(x).reshape(-1, 24)
    for i in range(x.shape[0]):
        d = float(blk[i, :2].view(np.float16)[0])
        m = float(blk[i, 2:4].view(np.float16)[0])
        xr = oracle.q5_1_decode(blk[i])
        bound = d / 2 * (1 + 2.0 ** -16) + abs(float(x[i].min()) - m)
        assert np.all(np.abs(x[i] - xr) <= bound), i


def test_quantize_rows_is_blockwise():
    x = _normal_blocks(12, 3).reshape(3, 128)
    kb = oracle.quantize_k(x)
    vb = oracle.quantize_v(x)
    for j in range(12):
        r, c = divmod(j, 4)
        assert np.array_equal(kb[34 * j:34 * j + 34], oracle.q8_0_encode(x[r, 32 * c:32 * c + 32]))
        assert np.array_equal(vb[24 * j:24 * j + 24], oracle.q5_1_encode(x[r, 32 * c:32 * c + 32]))


def test_q5_1_codes_in_range_and_monotone():
    x = np.sort(_normal_blocks(200, 4) * 1e-4, axis=1)   # includes subnormal-scale blocks
    for row in x:
        c = _unpack_q5_1(oracle.q5_1_encode(row))
        assert c.min() >= 0 and c.max() <= 31
        assert np.all(np.diff(c) >= 0)


def test_q5_1_zero_minimum_is_stored_as_positive_zero():
    x = np.zeros(32, np.float32)
    x[1::3] = -0.0
    x[2::5] = 2.5
    for arr in (x, x[::-1].copy(), np.full(32, -0.0, np.float32)):
        blk = oracle.q5_1_encode(arr)
        assert blk[2] == 0 and blk[3] == 0


def test_q5_1_negative_zero_block_has_positive_zero_step_and_offset():
    blk = oracle.q5_1_encode(np.full(32, -0.0, np.float32))
    assert np.array_equal(blk, np.zeros(24, np.uint8))
