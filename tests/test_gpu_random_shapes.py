"""Seeded random shapes through the C ABI against the oracle: head_dim from
32 to 256, 1 to 8 KV heads, 1 to 8 query heads per KV head, 1 to 40 query
rows, flat caches or windowed rings, with and without sinks, fp32 or bf16
inputs, ragged lengths and several appends per case; and FP8 (e4m3) rows at
head_dim 64, 128 and 256 with up to 96 query rows (prompt chunks on the
prime kernel among them).  Every case checks the stored bytes of every live
row and every output element."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

from gpu_pair import Pair  # noqa: E402
from test_gpu_parity import qrows, rows  # noqa: E402

N_CASES = 48


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    hd = int(rng.choice([32, 64, 96, 128, 160, 256]))
    Hkv = int(rng.integers(1, 9))
    hpk = int(rng.choice([1, 2, 3, 4, 5, 8]))
    B = int(rng.integers(1, 5))
    T = int(rng.choice([1, 1, 2, 3, 8, 13, 40]))
    io = "bf16" if rng.random() < 0.7 else "f32"
    ring = rng.random() < 0.35
    sinks = rng.random() < 0.5
    if ring:
        window = int(rng.integers(max(T, 16), 200))
        step = int(rng.choice([16, 32, 64]))
        cap = window + step + T + int(rng.integers(0, 64))
        lens = rng.integers(T, 3 * cap, size=B)
    else:
        window = int(rng.choice([0, 0, int(rng.integers(T, 300))]))
        step = 0
        lens = rng.integers(T, 900, size=B)
        cap = int(lens.max()) + T + 16
    return rng, dict(B=B, H=Hkv * hpk, Hkv=Hkv, hd=hd, T=T, io=io, window=window, step=step, cap=cap,
                     lens=lens.tolist(), sinks=sinks)


N_F8_CASES = 24


def draw_f8(seed):
    """FP8 rows: head_dim 64, 128 or 256, ring steps multiples of 32."""
    rng = np.random.default_rng(5000 + seed)
    hd = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.integers(1, 9))
    hpk = int(rng.choice([1, 2, 3, 4, 5, 8]))
    B = int(rng.integers(1, 4))
    T = int(rng.choice([1, 2, 8, 13, 40, 96]))
    io = "bf16" if rng.random() < 0.7 else "f32"
    ring = rng.random() < 0.35
    sinks = rng.random() < 0.5
    if ring:
        window = int(rng.integers(max(T, 16), 200))
        step = int(rng.choice([32, 64]))
        cap = window + step + T + 31 + int(rng.integers(0, 64))
        lens = rng.integers(T, 3 * cap, size=B)
    else:
        window = int(rng.choice([0, 0, int(rng.integers(T, 300))]))
        step = 0
        lens = rng.integers(T, 700, size=B)
        cap = int(lens.max()) + T + 16
    return rng, dict(B=B, H=Hkv * hpk, Hkv=Hkv, hd=hd, T=T, io=io, window=window, step=step, cap=cap,
                     lens=lens.tolist(), sinks=sinks)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape(seed):
    run_case(seed, *draw(seed))


@pytest.mark.parametrize("seed", range(N_F8_CASES))
def test_random_shape_f8(seed):
    run_case(seed, *draw_f8(seed), fmt="e4m3")


def run_case(seed, rng, c, fmt="q8_0/q5_1"):
    print(f"case {seed} {fmt}: {c}", flush=True)
    B, H, Hkv, hd, T, io = c["B"], c["H"], c["Hkv"], c["hd"], c["T"], c["io"]
    p = Pair(B, H, Hkv, hd, c["cap"], c["window"], c["step"], io=io, fmt=fmt)
    lens = np.asarray(c["lens"])
    done = np.zeros(B, np.int64)
    # pieces small enough for a ring's rebase rule (the first new row keeps
    # its window); the last append is the T query rows themselves, so that
    # every query row's window is still resident
    piece = max(1, c["cap"] - c["window"] - c["step"] + 1) if c["step"] else 500
    while np.any(done < lens - T):
        n = np.minimum(lens - T - done, rng.integers(1, piece + 1))
        k, v = rows(rng, B, int(n.max()), Hkv, hd, io, scale=float(rng.choice([0.25, 1.0])))
        p.append(k, v, n.tolist())
        done += n
    k, v = rows(rng, B, T, Hkv, hd, io)
    p.append(k, v)
    p.check_mirror()
    p.check_planes()
    q = qrows(rng, B, T, H, hd, io)
    s = (rng.standard_normal(H) * 2).astype(np.float32) if c["sinks"] else None
    p.decode(q, float(np.float32(1 / np.sqrt(hd))), sinks=s, what=f"case {seed} {fmt}")
