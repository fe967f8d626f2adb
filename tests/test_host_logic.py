"""Host logic of libkvq on the CPU: validation, host mirror, ring planner,
split-K plan and the "refuse, enqueue nothing, change nothing" rule.

libkvq_nodev.so is the same kvq_host.cpp linked to a launcher that records
each launch as a line of text instead of running it.  Device pointers are
plain 256-aligned integers that are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from decode_attention_quantized_append_amd import build, kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
K, V, C, Q, O, WS = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000, 0x60000000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvq.NODEV_PATH):
        build.build_nodev(verbose=False)
    return kvq.load_nodev()


def log(lib):
    return lib.kvq_nodev_log().decode().splitlines()


def fields(line):
    """key=integer fields of a recorded launch ("rows=a+b" gives rows=a)."""
    return {k: int(v) for k, v in re.findall(r"(\w+)=(-?\d+)", line)}


def create(lib, **kw):
    cfg = kvq.make_config(**{**dict(n_seqs=2, n_q_heads=8, n_kv_heads=2, head_dim=64, capacity=100), **kw})
    lib.kvq_nodev_clear()
    return kvq.kvq_create(cfg, K, V, C, 0, lib)


def err(lib, fn, *a):
    with pytest.raises(kvq.KvqError) as e:
        fn(*a, lib=lib)
    return e.value.status


def lengths(lib, h, B):
    return kvq.kvq_host_lengths(h, B, lib)


# -- header and exports ------------------------------------------------------
def test_header_declares_exactly_the_exports():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    declared = set(re.findall(r"^(?:kvq_status|void|const char\*)\s+(kvq_\w+)\(", text, re.M))
    assert declared == set(kvq.EXPORTS)


def test_nodev_library_exports_every_symbol(lib):
    for name in kvq.EXPORTS:
        assert hasattr(lib, name)


def test_hip_library_loads_and_exports_every_symbol():
    if not os.path.exists(kvq.LIB_PATH):
        build.build_hip(verbose=False)
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    syms = set(re.findall(r" T (kvq_\w+)", out))
    assert set(kvq.EXPORTS) <= syms
    lib = ctypes.CDLL(kvq.LIB_PATH)          # loads without a GPU; nothing is called
    for name in kvq.EXPORTS:
        assert hasattr(lib, name)


# -- sizes and create ---------------------------------------------------------
def test_required_bytes(lib):
    cfg = kvq.make_config(16, 40, 8, 128, 33000)
    s = kvq.kvq_required_bytes(cfg, lib)
    assert (s.k_row_bytes, s.v_row_bytes) == (32 * 34, 32 * 24) == (1088, 768)
    assert s.k_session_stride == -(-1088 * 33000 // 256) * 256
    assert s.k_planes_bytes == 16 * s.k_session_stride + 256 and s.v_planes_bytes == 16 * s.v_session_stride + 256
    assert s.counters_bytes >= (2 * 16 + 4) * 4 and s.counters_bytes % 256 == 0


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=48), kvq.KVQ_EINVAL), (dict(head_dim=0), kvq.KVQ_EINVAL),
    (dict(head_dim=288), kvq.KVQ_EUNSUPPORTED), (dict(n_q_heads=7), kvq.KVQ_EINVAL),
    (dict(n_seqs=0), kvq.KVQ_EINVAL), (dict(capacity=0), kvq.KVQ_EINVAL),
    (dict(ring_step=16), kvq.KVQ_EINVAL), (dict(window=90, ring_step=16), kvq.KVQ_EINVAL),
    (dict(window=-1), kvq.KVQ_EINVAL)])
def test_bad_config(lib, kw, status):
    cfg = kvq.make_config(**{**dict(n_seqs=2, n_q_heads=8, n_kv_heads=2, head_dim=64, capacity=100), **kw})
    assert err(lib, kvq.kvq_required_bytes, cfg) == status
    lib.kvq_nodev_clear()
    with pytest.raises(kvq.KvqError):
        kvq.kvq_create(cfg, K, V, C, 0, lib)
    assert log(lib) == []


def test_formats_other_than_q8_0_q5_1_are_unsupported(lib):
    cfg = kvq.make_config(1, 4, 1, 64, 10)
    cfg.v_fmt = kvq.KVQ_FMT_Q8_0
    assert err(lib, kvq.kvq_required_bytes, cfg) == kvq.KVQ_EUNSUPPORTED


def test_create_zeroes_counters_and_checks_alignment(lib):
    h = create(lib)
    assert log(lib) == ["set " + " ".join(f"{i}=0" for i in range(2 * 2 + 4))]
    cfg = kvq.make_config(2, 8, 2, 64, 100)
    lib.kvq_nodev_clear()
    for k, v, c in ((K + 8, V, C), (K, V + 128, C), (K, V, C + 4), (0, V, C)):
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_create(cfg, k, v, c, 0, lib)
        assert e.value.status == kvq.KVQ_EINVAL
    assert log(lib) == []
    kvq.kvq_destroy(h, lib)


# -- append ---------------------------------------------------------------------
def test_append_flat_and_capacity(lib):
    h = create(lib)
    lib.kvq_nodev_clear()
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 60, None, 0, lib)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 40, [40, 7], 0, lib)
    assert log(lib) == ["append b0=0 T=60 n=60,60", "append b0=0 T=40 n=40,7"]
    assert lengths(lib, h, 2) == ([100, 67], [0, 0])
    lib.kvq_nodev_clear()
    assert err(lib, kvq.kvq_append, h, Q, Q, kvq.KVQ_BF16, 1) == kvq.KVQ_ECAPACITY
    assert err(lib, kvq.kvq_append, h, Q, Q, kvq.KVQ_BF16, 2, [2, 3]) == kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_append, h, Q, Q, 7, 1) == kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_append, h, Q, Q, kvq.KVQ_F32, 0) == kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_append, h, 0, Q, kvq.KVQ_F32, 1) == kvq.KVQ_EINVAL
    assert log(lib) == [] and lengths(lib, h, 2) == ([100, 67], [0, 0])
    kvq.kvq_append(h, Q, Q, kvq.KVQ_F32, 5, [0, 5], 0, lib)     # session 0 appends nothing
    assert lengths(lib, h, 2)[0] == [100, 72]


def test_append_sessions_split_across_launches(lib):
    h = create(lib, n_seqs=70, capacity=10)
    lib.kvq_nodev_clear()
    kvq.kvq_append(h, Q, Q, kvq.KVQ_F32, 2, [1] * 64 + [2] * 6, 0, lib)
    assert log(lib) == ["append b0=0 T=2 n=" + ",".join(["1"] * 64), "append b0=64 T=2 n=2,2,2,2,2,2"]


def test_ring_rebase_plan_matches_the_oracle_cache_model(lib):
    from oracle.cache_model import OracleCache
    B, cap, W, step = 3, 16, 8, 4
    h = create(lib, n_seqs=B, capacity=cap, window=W, ring_step=step)
    model = OracleCache(B, 2, 64, cap, window=W, ring_step=step)
    rng = np.random.default_rng(0)
    for _ in range(40):
        n = rng.integers(0, 6, size=B)
        T = int(n.max()) or 1
        lib.kvq_nodev_clear()
        before = lengths(lib, h, B)
        kvq.kvq_append(h, Q, Q, kvq.KVQ_F32, T, n.tolist(), 0, lib)
        z = np.zeros((B, T, 2, 64), np.float32)
        model.append(z, z, n)
        after = lengths(lib, h, B)
        assert after == (model.len.tolist(), model.base.tolist())
        # every rebase is a sequence of non-overlapping slabs, then the base_d write
        moved = [ln for ln in log(lib) if ln.startswith("move")]
        for b in range(B):
            shift = after[1][b] - before[1][b]
            if shift == 0:
                continue
            keep = before[0][b] - after[1][b]
            slabs = [tuple(map(int, re.match(r"(\d+):(\d+)>(\d+)x(\d+)", tok).groups()))
                     for ln in moved for tok in ln.split()[1:] if tok.startswith(f"{b}:")]
            covered = 0
            for (_, src, dst, rows) in slabs:
                assert src == dst + shift and rows <= shift and dst == covered
                covered += rows
            assert covered == keep
            assert f"{B + b}={after[1][b]}" in [t for ln in log(lib) if ln.startswith("set") for t in ln.split()]


def test_registered_importance_moves_with_the_rows(lib):
    """With an importance array registered, every rebase slab moves its
    entries too, and the positions past the survivors are cleared."""
    B, cap, W, step = 2, 16, 8, 4
    h = create(lib, n_seqs=B, capacity=cap, window=W, ring_step=step)
    kvq.kvq_set_importance(h, 0x70000000, lib)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_F32, 14, [14, 9], 0, lib)
    lib.kvq_nodev_clear()
    kvq.kvq_append(h, Q, Q, kvq.KVQ_F32, 3, None, 0, lib)      # session 0: 17 rows > 16 -> base 4
    lines = log(lib)
    moves = [ln for ln in lines if ln.startswith("move")]
    assert moves and all(ln.startswith("move+imp ") for ln in moves)
    (zero,) = [ln for ln in lines if ln.startswith("zero_imp")]
    assert zero == "zero_imp 0@10+6"                               # 14 - 4 survivors
    assert lines.index(zero) > max(lines.index(m) for m in moves)
    assert lengths(lib, h, B) == ([17, 12], [4, 0])
    kvq.kvq_set_importance(h, None, lib)
    lib.kvq_nodev_clear()
    kvq.kvq_append(h, Q, Q, kvq.KVQ_F32, 14, [4, 0], 0, lib)      # session 0: 21 rows -> base 8
    lines = log(lib)
    assert [ln for ln in lines if ln.startswith("move ")] and lengths(lib, h, B) == ([21, 12], [8, 0])
    assert not [ln for ln in lines if ln.startswith(("move+imp", "zero_imp"))]
    assert err(lib, kvq.kvq_set_importance, h, 0x70000002) == kvq.KVQ_EINVAL


def test_ring_refuses_to_drop_visible_rows(lib):
    h = create(lib, n_seqs=1, capacity=16, window=8, ring_step=4)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_F32, 14, None, 0, lib)
    lib.kvq_nodev_clear()
    assert err(lib, kvq.kvq_append, h, Q, Q, kvq.KVQ_F32, 9) == kvq.KVQ_ERANGE
    assert log(lib) == [] and lengths(lib, h, 1) == ([14], [0])


# -- truncate -------------------------------------------------------------------
def test_truncate(lib):
    h = create(lib)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_F32, 50, None, 0, lib)
    lib.kvq_nodev_clear()
    kvq.kvq_truncate(h, [47, 50], 0, lib)
    assert log(lib) == ["set 0=47"] and lengths(lib, h, 2)[0] == [47, 50]
    lib.kvq_nodev_clear()
    assert err(lib, kvq.kvq_truncate, h, [48, 50]) == kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_truncate, h, [-1, 50]) == kvq.KVQ_EINVAL
    assert log(lib) == []


def test_truncate_never_moves_base_and_guards_the_window(lib):
    h = create(lib, n_seqs=1, capacity=16, window=8, ring_step=4)
    for _ in range(30):
        kvq.kvq_append(h, Q, Q, kvq.KVQ_F32, 1, None, 0, lib)
    L, base = lengths(lib, h, 1)
    assert base[0] > 0
    lib.kvq_nodev_clear()
    kvq.kvq_truncate(h, [base[0] + 8], 0, lib)
    assert lengths(lib, h, 1) == ([base[0] + 8], base)
    assert err(lib, kvq.kvq_truncate, h, [base[0] + 7]) == kvq.KVQ_ERANGE
    assert all(not ln.startswith("move") for ln in log(lib))


# -- decode -----------------------------------------------------------------------
def test_decode_validation_and_plan(lib):
    h = create(lib, n_seqs=2, capacity=5000)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 3000, [3000, 1000], 0, lib)
    ws = kvq.kvq_decode_workspace_bytes(h, 2, lib)
    lib.kvq_nodev_clear()
    kvq.kvq_decode(h, Q, kvq.KVQ_BF16, 2, None, 0.125, O, None, WS, ws, 0, lib)
    (line,) = log(lib)
    chunk, splits = map(int, re.search(r"chunk=(\d+) splits=(\d+)", line).groups())
    assert chunk % 32 == 0 and splits == -(-3000 // chunk)
    ml = int(re.search(r"ml_to_o=(\d+)", line).group(1))
    assert ml >= 2 * splits * 2 * 8 * 4 and ml % 256 == 0
    assert ws >= ml + 2 * splits * 2 * 8 * 64 * 4
    lib.kvq_nodev_clear()
    assert err(lib, kvq.kvq_decode, h, Q, kvq.KVQ_BF16, 2, None, 0.125, O, None, WS, ws - 1) == kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_decode, h, Q, kvq.KVQ_BF16, 2, None, 0.125, O, None, WS + 16, ws) == kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_decode, h, Q, kvq.KVQ_BF16, 1001, None, 0.125, O, None, WS, 1 << 40) == kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_decode, h, Q, kvq.KVQ_BF16, 2, None, float("nan"), O, None, WS, ws) == kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_decode, h, 0, kvq.KVQ_BF16, 2, None, 0.125, O, None, WS, ws) == kvq.KVQ_EINVAL
    kvq.kvq_truncate(h, [3000, 1], 0, lib)
    lib.kvq_nodev_clear()
    assert err(lib, kvq.kvq_decode, h, Q, kvq.KVQ_BF16, 2, None, 0.125, O, None, WS, 1 << 40) == kvq.KVQ_EINVAL
    assert log(lib) == []


def test_decode_query_row_groups(lib):
    # more than 32 query rows per KV head: the decode workgroups take groups
    # of 32 / hpk rows (the launch's y index), and the combine folds all T
    h = create(lib, n_seqs=2, n_q_heads=8, n_kv_heads=2, head_dim=64, capacity=5000)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 3000, [3000, 1000], 0, lib)
    ws = kvq.kvq_decode_workspace_bytes(h, 20, lib)
    lib.kvq_nodev_clear()
    kvq.kvq_decode(h, Q, kvq.KVQ_BF16, 20, None, 0.125, O, None, WS, ws, 0, lib)
    (line,) = log(lib)
    r = fields(line)
    assert (r["T"], r["Tg"], r["groups"]) == (20, 8, 3)
    assert ws >= r["ml_to_o"] + 2 * r["splits"] * 20 * 8 * 64 * 4   # partials of all 20 rows
    assert r["ml_to_o"] >= 2 * r["splits"] * 20 * 8 * 2 * 4
    # the same plan as one group of 8 rows
    lib.kvq_nodev_clear()
    kvq.kvq_decode(h, Q, kvq.KVQ_BF16, 8, None, 0.125, O, None, WS, ws, 0, lib)
    (line8,) = log(lib)
    r8 = fields(line8)
    assert (r8["Tg"], r8["groups"]) == (8, 1)
    assert all(r8[k] == r[k] for k in ("chunk", "splits", "kernel", "gh", "rs", "rg", "units"))


def test_graph_mode_plan_and_host_resync(lib):
    # graph mode: the decode plan covers each session's largest span (the
    # plane, or the window plus T - 1 plus 31 rows), whatever the lengths now
    h = create(lib, n_seqs=2, capacity=5000)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 3000, [3000, 1000], 0, lib)
    now = plan_of(lib, h)
    kvq.kvq_set_graph_mode(h, True, lib)
    g = plan_of(lib, h)
    assert g["splits"] == -(-5000 // g["chunk"]) and g["units"] == 2 * g["splits"]
    assert g["units"] >= now["units"]
    assert kvq.kvq_decode_workspace_bytes(h, 1, lib) >= (g["ml_to_o"] + 2 * g["splits"] * 8 * 64 * 4)
    kvq.kvq_set_graph_mode(h, False, lib)
    assert plan_of(lib, h) == now
    assert lib.kvq_set_graph_mode(h, 2) == kvq.KVQ_EINVAL
    hw = create(lib, n_seqs=1, capacity=4096, window=100, ring_step=512)
    kvq.kvq_append(hw, Q, Q, kvq.KVQ_BF16, 50, None, 0, lib)
    kvq.kvq_set_graph_mode(hw, True, lib)
    pw = plan_of(lib, hw, T=3)
    assert pw["splits"] == -(-(100 + 2 + 31) // pw["chunk"])
    # the host mirror set from outside (after replays the host did not see)
    lib.kvq_nodev_clear()
    kvq.kvq_set_host_lengths(h, [3100, 1200], [0, 0], lib)
    assert lengths(lib, h, 2) == ([3100, 1200], [0, 0])
    assert log(lib) == []
    assert err(lib, kvq.kvq_set_host_lengths, h, [5001, 10], [0, 0]) == kvq.KVQ_EINVAL   # past the plane
    assert err(lib, kvq.kvq_set_host_lengths, h, [10, 10], [0, 11]) == kvq.KVQ_EINVAL    # base above len
    assert err(lib, kvq.kvq_set_host_lengths, h, [10, 10], [0, 5]) == kvq.KVQ_EINVAL     # flat: base 0
    assert lengths(lib, h, 2) == ([3100, 1200], [0, 0])
    kvq.kvq_set_host_lengths(hw, [5000], [4000], lib)
    assert lengths(lib, hw, 1) == ([5000], [4000])


def test_importance_launch(lib):
    # one launch over the 16-row tiles of the longest span of visible rows
    h = create(lib, n_seqs=2, capacity=5000)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 3000, [3000, 1000], 0, lib)
    lib.kvq_nodev_clear()
    kvq.kvq_importance(h, Q, kvq.KVQ_BF16, 2, 0.1, O, O, 0, lib)
    (line,) = log(lib)
    assert fields(line)["tiles"] == -(-3000 // 16) and fields(line)["T"] == 2
    # K rows of 2 heads x 64 dims: 136 bytes, 11 pieces of LDS each (odd, with
    # room for a row starting up to 15 bytes into its first piece); 64 rows
    assert fields(line)["rp"] == 11 and fields(line)["group_rows"] == 64
    lib.kvq_nodev_clear()
    assert err(lib, kvq.kvq_importance, h, Q, kvq.KVQ_BF16, 1001, 0.1, O, O) == kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_importance, h, Q, kvq.KVQ_BF16, 1, 0.1, O, 0) == kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_importance, h, Q, 7, 1, 0.1, O, O) == kvq.KVQ_EINVAL
    assert log(lib) == []
    hw = create(lib, n_seqs=1, capacity=300, window=100, ring_step=50)
    for _ in range(6):
        kvq.kvq_append(hw, Q, Q, kvq.KVQ_BF16, 40, None, 0, lib)
    lib.kvq_nodev_clear()
    kvq.kvq_importance(hw, Q, kvq.KVQ_BF16, 3, 0.1, O, O, 0, lib)
    assert fields(log(lib)[0])["tiles"] == -(-(100 + 2) // 16)
    # long rows: 37 KV heads x 256 dims (10064-byte rows) leave room for 16
    # rows in the whole LDS; 38 heads x 256 not even for that
    hl = create(lib, n_seqs=1, n_q_heads=37, n_kv_heads=37, head_dim=256, capacity=64)
    kvq.kvq_append(hl, Q, Q, kvq.KVQ_BF16, 20, None, 0, lib)
    lib.kvq_nodev_clear()
    kvq.kvq_importance(hl, Q, kvq.KVQ_BF16, 1, 0.1, O, O, 0, lib)
    f = fields(log(lib)[0])
    assert f["rp"] == 631 and f["group_rows"] == 16
    hx = create(lib, n_seqs=1, n_q_heads=38, n_kv_heads=38, head_dim=256, capacity=64)
    kvq.kvq_append(hx, Q, Q, kvq.KVQ_BF16, 20, None, 0, lib)
    lib.kvq_nodev_clear()
    assert err(lib, kvq.kvq_importance, hx, Q, kvq.KVQ_BF16, 1, 0.1, O, O) == kvq.KVQ_EUNSUPPORTED
    assert log(lib) == []


def test_rollback_relative(lib):
    # a rollback enqueues len_d -= drop (relative, so a captured round can be
    # replayed) and moves the host mirror by the same amount
    h = create(lib, n_seqs=3, capacity=500)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 40, [40, 30, 10], 0, lib)
    lib.kvq_nodev_clear()
    kvq.kvq_rollback(h, [5, 0, 10], 0, lib)
    assert log(lib) == ["add 0=-5 2=-10"]
    assert lengths(lib, h, 3) == ([35, 30, 0], [0, 0, 0])
    lib.kvq_nodev_clear()
    assert err(lib, kvq.kvq_rollback, h, [36, 0, 0]) == kvq.KVQ_EINVAL     # past zero
    assert err(lib, kvq.kvq_rollback, h, [-1, 0, 0]) == kvq.KVQ_EINVAL
    assert log(lib) == [] and lengths(lib, h, 3) == ([35, 30, 0], [0, 0, 0])
    # a windowed ring refuses to expose rows it no longer holds
    hw = create(lib, n_seqs=1, capacity=16, window=8, ring_step=4)
    for _ in range(30):
        kvq.kvq_append(hw, Q, Q, kvq.KVQ_F32, 1, None, 0, lib)
    L, base = lengths(lib, hw, 1)
    ok = L[0] - 8 - base[0]                       # rows that can go before the window leaves the ring
    lib.kvq_nodev_clear()
    assert err(lib, kvq.kvq_rollback, hw, [ok + 1]) == kvq.KVQ_ERANGE
    kvq.kvq_rollback(hw, [ok], 0, lib)
    assert lengths(lib, hw, 1)[0] == [L[0] - ok]


def test_decode_query_tile_limits(lib):
    h = create(lib, n_seqs=1, n_q_heads=64, n_kv_heads=1, head_dim=256, capacity=100)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 50, None, 0, lib)
    # 64 query rows per KV head exceed the 32 that kvq_decode accepts (EINVAL, as declared)
    assert err(lib, kvq.kvq_decode, h, Q, kvq.KVQ_BF16, 1, None, 0.1, O, None, WS, 1 << 40) == kvq.KVQ_EINVAL


def test_decode_refuses_rebased_rows(lib):
    h = create(lib, n_seqs=1, capacity=16, window=8, ring_step=4)
    for _ in range(30):
        kvq.kvq_append(h, Q, Q, kvq.KVQ_F32, 1, None, 0, lib)
    L, base = lengths(lib, h, 1)
    ok_T = L[0] - 8 + 1 - base[0]      # largest T whose first row's window is resident
    kvq.kvq_decode(h, Q, kvq.KVQ_F32, ok_T, None, 0.1, O, None, WS, 1 << 40, 0, lib)
    assert err(lib, kvq.kvq_decode, h, Q, kvq.KVQ_F32, ok_T + 1, None, 0.1, O, None, WS, 1 << 40) == kvq.KVQ_ERANGE


def test_split_rows_setting(lib):
    h = create(lib, n_seqs=1, capacity=5000)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_F32, 4000, None, 0, lib)
    assert err(lib, kvq.kvq_set_split_rows, h, 100) == kvq.KVQ_EINVAL
    kvq.kvq_set_split_rows(h, 640, lib)
    lib.kvq_nodev_clear()
    kvq.kvq_decode(h, Q, kvq.KVQ_F32, 1, None, 0.1, O, None, WS, 1 << 40, 0, lib)
    assert "chunk=640 splits=7" in log(lib)[0]
    assert kvq.kvq_info(h, lib).split_rows == 640


def plan_of(lib, h, T=1, dtype=kvq.KVQ_BF16):
    lib.kvq_nodev_clear()
    kvq.kvq_decode(h, Q, dtype, T, None, 0.1, O, None, WS, 1 << 40, 0, lib)
    (line,) = log(lib)
    return {k: int(v) for k, v in re.findall(r"(\w+)=(-?\d+)", line)}


def test_decode_kernel_choice(lib):
    PER_HEAD, STREAM = 0, 2                        # as recorded by the launcher
    # 8 KV heads x 128: one wave per KV head; 8192 rows would give each wave a
    # single tile with 8 heads per workgroup, so 4 heads per workgroup take
    # two tiles each (64-row chunks, the same number of workgroups)
    h = create(lib, n_seqs=1, n_q_heads=32, n_kv_heads=8, head_dim=128, capacity=9000)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 8192, None, 0, lib)
    p = plan_of(lib, h)
    assert (p["kernel"], p["gh"], p["chunk"]) == (STREAM, 4, 64) and 0 < p["lds"] <= 160 * 1024
    assert p["splits"] == -(-8192 // p["chunk"]) == p["units"]
    assert p["rs"] == 1
    # a head group that is set is kept
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_STREAM, 8, 0, lib)
    p = plan_of(lib, h)
    assert (p["kernel"], p["gh"], p["chunk"]) == (STREAM, 8, 32)
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_AUTO, 0, 0, lib)
    # longer sessions: chunks of several tiles, all heads of a row in one workgroup
    h2 = create(lib, n_seqs=4, n_q_heads=32, n_kv_heads=8, head_dim=128, capacity=30000)
    kvq.kvq_append(h2, Q, Q, kvq.KVQ_BF16, 20000, None, 0, lib)
    p = plan_of(lib, h2, dtype=kvq.KVQ_F32)
    assert (p["kernel"], p["gh"]) == (STREAM, 8) and p["chunk"] > 64
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_PER_HEAD, 0, 0, lib)
    assert plan_of(lib, h)["kernel"] == PER_HEAD
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_STREAM, 2, 0, lib)
    p = plan_of(lib, h)
    assert (p["kernel"], p["gh"]) == (STREAM, 2)
    E = kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_set_decode_tiling, h, kvq.KVQ_DECODE_STREAM, 3, 0) == E      # does not divide 8
    assert err(lib, kvq.kvq_set_decode_tiling, h, kvq.KVQ_DECODE_STREAM, 2, 4) == E      # 1 .. 3 waves per head
    assert err(lib, kvq.kvq_set_decode_tiling, h, kvq.KVQ_DECODE_PER_HEAD, 2, 0) == E    # no head groups there
    assert err(lib, kvq.kvq_set_decode_tiling, h, 2, 0, 0) == E                          # no kernel 2
    assert err(lib, kvq.kvq_set_decode_tiling, h, 5, 0, 0) == E
    # two row streams of fp32 queries are not built: that call fails, enqueueing nothing
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_STREAM, 8, 2, lib)
    lib.kvq_nodev_clear()
    assert err(lib, kvq.kvq_decode, h, Q, kvq.KVQ_F32, 1, None, 0.1, O, None, WS, 1 << 40) == E
    assert log(lib) == []
    # verify rows (T=8, 4 query heads per KV head: 32 rows): two waves per
    # 256-dim head, each half of its dims, one head per workgroup
    h = create(lib, n_seqs=2, n_q_heads=16, n_kv_heads=4, head_dim=256, capacity=5000)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 4000, None, 0, lib)
    p = plan_of(lib, h, T=8)
    assert (p["kernel"], p["gh"], p["ds"], p["rg"]) == (STREAM, 1, 2, 1) and 4 * p["lds"] <= 160 * 1024
    # FP8 rows: two heads per workgroup (their waves share the pieces of a
    # row's scale area); with verify-length rows also two row streams
    for cap, rs in ((5000, 1), (140000, 2)):
        hf = create(lib, n_seqs=2, n_q_heads=16, n_kv_heads=4, head_dim=256, capacity=cap, fmt="e4m3")
        kvq.kvq_append(hf, Q, Q, kvq.KVQ_BF16, cap - 100, None, 0, lib)
        p = plan_of(lib, hf, T=8)
        assert (p["kernel"], p["gh"], p["ds"], p["rs"]) == (STREAM, 2, 2, rs) and p["lds"] <= 160 * 1024
    hf = create(lib, n_seqs=2, n_q_heads=16, n_kv_heads=4, head_dim=128, capacity=900, fmt="e4m3")
    kvq.kvq_append(hf, Q, Q, kvq.KVQ_BF16, 500, None, 0, lib)
    assert (plan_of(lib, hf, T=8)["gh"], plan_of(lib, hf, T=8)["ds"]) == (2, 2)
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_STREAM, 4, 3, lib)
    p = plan_of(lib, h, T=8)
    assert (p["kernel"], p["gh"], p["ds"]) == (STREAM, 4, 2) and p["lds"] <= 160 * 1024
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_STREAM, 0, 2, lib)        # two 16-row groups instead
    p = plan_of(lib, h, T=8)
    assert (p["kernel"], p["gh"], p["ds"], p["rg"]) == (STREAM, 4, 1, 2) and p["lds"] <= 160 * 1024
    # dim halves need 17..32 rows of 256-dim heads
    lib.kvq_nodev_clear()
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_STREAM, 0, 3, lib)
    assert err(lib, kvq.kvq_decode, h, Q, kvq.KVQ_BF16, 4, None, 0.1, O, None, WS, 1 << 40) == E
    assert log(lib) == []
    # head_dim 96 has no stream kernel
    h = create(lib, n_seqs=1, n_q_heads=8, n_kv_heads=8, head_dim=96, capacity=100)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 50, None, 0, lib)
    assert plan_of(lib, h)["kernel"] == PER_HEAD
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_STREAM, 0, 0, lib)
    assert err(lib, kvq.kvq_decode, h, Q, kvq.KVQ_BF16, 1, None, 0.1, O, None, WS, 1 << 40) == E
    # a single KV head of 64: one wave per workgroup
    h = create(lib, n_seqs=1, n_q_heads=4, n_kv_heads=1, head_dim=64, capacity=300)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 256, None, 0, lib)
    p = plan_of(lib, h)
    assert (p["kernel"], p["gh"]) == (STREAM, 1) and p["chunk"] % 32 == 0


def test_decode_row_streams(lib):
    STREAM = 2
    # long sessions: two row streams per head (16 waves per workgroup) for
    # bf16 queries; fp32 queries need more registers and keep one
    h = create(lib, n_seqs=4, n_q_heads=40, n_kv_heads=8, head_dim=128, capacity=31000)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 30000, None, 0, lib)
    p = plan_of(lib, h)
    assert (p["kernel"], p["gh"], p["rs"]) == (STREAM, 8, 2) and p["lds"] <= 160 * 1024
    assert p["units"] == 4 * -(-30000 // p["chunk"]) <= 256
    assert plan_of(lib, h, dtype=kvq.KVQ_F32)["rs"] == 1
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_STREAM, 8, 1, lib)
    assert plan_of(lib, h)["rs"] == 1
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_STREAM, 8, 2, lib)
    assert plan_of(lib, h)["rs"] == 2
    lib.kvq_nodev_clear()
    assert err(lib, kvq.kvq_decode, h, Q, kvq.KVQ_F32, 1, None, 0.1, O, None, WS, 1 << 40) == kvq.KVQ_EINVAL
    # more than 16 query rows per KV head: sub_tiles 2 gives each 16-row
    # group its own wave, 1 keeps two row tiles in one wave; at head_dim 256
    # the default is 3, two waves each taking half of the dims
    h = create(lib, n_seqs=2, n_q_heads=16, n_kv_heads=4, head_dim=256, capacity=5000)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 4000, None, 0, lib)
    p = plan_of(lib, h, T=8)
    assert (p["kernel"], p["gh"], p["rs"], p["rg"], p["ds"]) == (STREAM, 1, 1, 1, 2)
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_STREAM, 0, 2, lib)
    p = plan_of(lib, h, T=8)
    assert (p["kernel"], p["gh"], p["rs"], p["rg"], p["ds"]) == (STREAM, 4, 1, 2, 1) and p["lds"] <= 160 * 1024
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_STREAM, 4, 1, lib)
    assert plan_of(lib, h, T=8)["rg"] == 1
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_STREAM, 2, 2, lib)
    assert (plan_of(lib, h, T=8)["rg"], plan_of(lib, h, T=1)["rg"]) == (2, 1)


def test_decode_prime_choice(lib):
    """Prompt chunks (four or more groups of 32 / hpk query rows per KV head):
    the prime kernel, one workgroup of eight row groups per (session, chunk,
    KV head) and block of eight groups, about one workgroup per CU; q8_0 /
    q5_1 at head_dim 64 and 128 only."""
    STREAM, PRIME = 2, 3
    lib.kvq_nodev_set_cus(256)
    h = create(lib, n_seqs=1, n_q_heads=32, n_kv_heads=8, head_dim=128, capacity=9000)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 8192, None, 0, lib)
    p = plan_of(lib, h, T=512)
    assert (p["kernel"], p["gh"], p["Tg"], p["groups"], p["lds"]) == (PRIME, 1, 8, 64, 109824)
    assert p["chunk"] % 32 == 0 and p["units"] == p["splits"] == -(-8192 // p["chunk"])
    assert p["units"] * 8 * 8 <= 256 < -(-8192 // (p["chunk"] - 32)) * 8 * 8   # one round, no smaller chunk
    assert plan_of(lib, h, T=25)["kernel"] == PRIME          # 4 groups
    assert plan_of(lib, h, T=24)["kernel"] == STREAM         # 3 groups
    assert plan_of(lib, h, T=24, dtype=kvq.KVQ_F32)["kernel"] == STREAM
    # set explicitly: any shape with two or more groups
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_PRIME, 0, 0, lib)
    assert plan_of(lib, h, T=9)["kernel"] == PRIME
    lib.kvq_nodev_clear()
    E = kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_decode, h, Q, kvq.KVQ_BF16, 8, None, 0.1, O, None, WS, 1 << 40) == E   # one group
    assert log(lib) == []
    assert err(lib, kvq.kvq_set_decode_tiling, h, kvq.KVQ_DECODE_PRIME, 2, 0) == E
    assert err(lib, kvq.kvq_set_decode_tiling, h, kvq.KVQ_DECODE_PRIME, 0, 1) == E
    # head_dim 64: a smaller layout; FP8 rows: raw tiles of codes plus a
    # 16-byte scale piece per row; 256: the stream kernel
    h = create(lib, n_seqs=2, n_q_heads=16, n_kv_heads=4, head_dim=64, capacity=3000)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 2000, None, 0, lib)
    p = plan_of(lib, h, T=100, dtype=kvq.KVQ_F32)
    assert (p["kernel"], p["lds"], p["groups"]) == (PRIME, 59520, 13)
    for hd, lds in ((128, 112896), (64, 62592)):
        h = create(lib, n_seqs=1, n_q_heads=32, n_kv_heads=8, head_dim=hd, capacity=3000, fmt="e4m3")
        kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 2000, None, 0, lib)
        p = plan_of(lib, h, T=200)
        assert (p["kernel"], p["lds"]) == (PRIME, lds)
    for kw in (dict(head_dim=256, n_q_heads=16, n_kv_heads=4),):
        h = create(lib, n_seqs=1, capacity=3000, **kw)
        kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 2000, None, 0, lib)
        assert plan_of(lib, h, T=200)["kernel"] == STREAM
        kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_PRIME, 0, 0, lib)
        lib.kvq_nodev_clear()
        assert err(lib, kvq.kvq_decode, h, Q, kvq.KVQ_BF16, 200, None, 0.1, O, None, WS, 1 << 40) == E
        assert log(lib) == []


def test_decode_ring_start_below_base_falls_back(lib):
    # ring_step 10: base is not always a multiple of 32, and the stream
    # kernel, which starts at the first visible row rounded down to 32, is
    # used only while that row is still resident
    h = create(lib, n_seqs=1, n_q_heads=32, n_kv_heads=8, head_dim=128, capacity=100, window=90,
               ring_step=10)
    for kernel, gh, want in ((kvq.KVQ_DECODE_STREAM, 8, 2), (kvq.KVQ_DECODE_AUTO, 0, 2)):
        kvq.kvq_set_decode_tiling(h, kernel, gh, 0, lib)
        seen = set()
        for _ in range(150):
            kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 1, None, 0, lib)
            L, base = lengths(lib, h, 1)
            lo = max(0, L[0] - 90)
            k = plan_of(lib, h)["kernel"]
            assert k == (want if (lo & ~31) >= base[0] else 0)
            seen.add(k)
        assert seen == {0, want}
    # the prime kernel (two groups of 8 rows here, set explicitly) falls back the same way
    h = create(lib, n_seqs=1, n_q_heads=32, n_kv_heads=8, head_dim=128, capacity=120, window=90,
               ring_step=10)
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_PRIME, 0, 0, lib)
    seen = set()
    for _ in range(150):
        kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 1, None, 0, lib)
        L, base = lengths(lib, h, 1)
        if L[0] < 9:
            continue
        k = plan_of(lib, h, T=9)["kernel"]
        assert k == (3 if (max(0, L[0] - 98) & ~31) >= base[0] else 0)
        seen.add(k)
    assert seen == {0, 3}


def _ring_model_ok(cap, W, C, S):
    """The rebase rule kvq_append documents, over every session state reachable
    from empty by appends of 1..C rows: True when no append drops a row its
    first new row sees and no decode start (first visible row rounded down to
    32) lies below base."""
    if W + S > cap:
        return False
    seen, stack = {(0, 0)}, [(0, 0)]
    while stack:
        L, b = stack.pop()
        for n in range(1, C + 1):
            nb = b
            while L + n - nb > cap:
                nb += S
            lo = max(0, L + 1 - W)
            if (nb != b and lo < nb) or (lo & ~31) < nb:
                return False
            st = (L + n, nb)
            if st[0] <= 4 * cap + 100 and st not in seen:
                seen.add(st)
                stack.append(st)
    return True


@pytest.mark.parametrize("W,C,S", [(64, 32, 32), (64, 40, 32), (64, 16, 64), (128, 64, 96), (100, 33, 48),
                                   (96, 64, 40), (50, 20, 17), (80, 7, 5), (40, 1, 32)])
def test_ring_rows_formula_against_the_rebase_rule(lib, W, C, S):
    rows = kvq.kvq_ring_rows(W, C, S, lib)
    assert rows == max(W + S, W + C + S - 2 + (0 if S % 32 == 0 else 31))
    assert _ring_model_ok(rows, W, C, S)
    if S % 32 == 0 and rows > W + S:
        assert not _ring_model_ok(rows - 1, W, C, S)      # the smallest such ring


def test_ring_rows_serves_prime_chunks_from_the_ring(lib):
    """Random prompt chunks of up to C rows, then single rows, appended to a
    ring of kvq_ring_rows rows: no append fails and every decode of the
    appended rows runs the stream kernel (its 32-aligned start is resident)."""
    rng = np.random.default_rng(5)
    for W, C, S in ((96, 40, 32), (90, 33, 10), (256, 128, 64)):
        cap = kvq.kvq_ring_rows(W, C, S, lib)
        h = create(lib, n_seqs=1, n_q_heads=32, n_kv_heads=8, head_dim=128, capacity=cap, window=W, ring_step=S)
        for i in range(120):
            n = int(rng.integers(1, C + 1)) if i < 80 else 1
            kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, n, None, 0, lib)
            L, base = lengths(lib, h, 1)
            assert ((max(0, L[0] - n + 1 - W)) & ~31) >= base[0]
            # the stream kernel, or from four groups of 8 rows on the prime kernel
            assert plan_of(lib, h, T=n)["kernel"] == (3 if n > 24 else 2)
        kvq.kvq_destroy(h, lib)
    from decode_attention_quantized_append_amd import workloads
    w = workloads.get("prime")
    assert w.ring_cap == kvq.kvq_ring_rows(w.window, w.T, w.ring_step, lib)
    assert err(lib, kvq.kvq_ring_rows, 0, 8, 32) == kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_ring_rows, 64, 0, 32) == kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_ring_rows, 64, 8, 0) == kvq.KVQ_EINVAL
    assert err(lib, kvq.kvq_ring_rows, 2 ** 31 - 1, 8, 32) == kvq.KVQ_EINVAL


def test_launch_failure_reports_edevice_and_keeps_the_mirror(lib):
    h = create(lib)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_F32, 10, None, 0, lib)
    lib.kvq_nodev_fail_next()
    assert err(lib, kvq.kvq_truncate, h, [5, 5]) == kvq.KVQ_EDEVICE
    assert lengths(lib, h, 2)[0] == [10, 10]
    lib.kvq_nodev_fail_next()
    assert err(lib, kvq.kvq_append, h, Q, Q, kvq.KVQ_F32, 1) == kvq.KVQ_EDEVICE
    assert lengths(lib, h, 2)[0] == [10, 10]
    assert "simulated" in kvq.kvq_last_error(lib)


def test_info(lib):
    h = create(lib, n_seqs=3, capacity=77, window=5)
    info = kvq.kvq_info(h, lib)
    assert (info.config.n_seqs, info.config.capacity, info.config.window) == (3, 77, 5)
    assert (info.k_planes, info.v_planes, info.counters) == (K, V, C)


def test_plan_follows_the_device_compute_units(lib):
    """One round of decode workgroups is sized to the CUs of the device the
    handle was created on (read at kvq_create), not to a fixed count."""
    chunks = {}
    try:
        for cus in (256, 128, 64):
            lib.kvq_nodev_set_cus(cus)
            h = create(lib, n_seqs=4, n_q_heads=40, n_kv_heads=8, head_dim=128, capacity=31000)
            kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 30000, None, 0, lib)
            p = plan_of(lib, h)
            chunks[cus] = p["chunk"]
            assert p["units"] * (8 // p["gh"]) <= cus * 8   # at most one round of workgroups
        assert chunks[256] < chunks[128] < chunks[64]
        lib.kvq_nodev_set_cus(0)                             # an unreadable count: no handle
        cfg = kvq.make_config(1, 4, 1, 64, 100)
        out = ctypes.c_void_p()
        assert lib.kvq_create(ctypes.byref(cfg), K, V, C, None, ctypes.byref(out)) == kvq.KVQ_EDEVICE
    finally:
        lib.kvq_nodev_set_cus(256)


def test_trace_events_are_recorded_around_the_decode_kernels(lib):
    """kvq_set_trace_events: later decodes record the caller's events (the
    recording launcher marks such a launch), NULL stops it; nothing else
    changes."""
    h = create(lib, n_seqs=1, n_q_heads=8, n_kv_heads=2, head_dim=64, capacity=300)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 100, None, 0, lib)
    lib.kvq_nodev_clear()
    kvq.kvq_decode(h, Q, kvq.KVQ_BF16, 1, None, 0.1, O, None, WS, 1 << 40, 0, lib)
    plain = log(lib)[0]
    kvq.kvq_set_trace_events(h, 0x1000, 0x2000, 0x3000, lib)
    lib.kvq_nodev_clear()
    kvq.kvq_decode(h, Q, kvq.KVQ_BF16, 1, None, 0.1, O, None, WS, 1 << 40, 0, lib)
    (traced,) = log(lib)
    assert traced == "traced " + plain
    kvq.kvq_set_trace_events(h, None, None, None, lib)
    lib.kvq_nodev_clear()
    kvq.kvq_decode(h, Q, kvq.KVQ_BF16, 1, None, 0.1, O, None, WS, 1 << 40, 0, lib)
    assert log(lib) == [plain]
    assert err(lib, kvq.kvq_set_trace_events, None, None, None, None) == kvq.KVQ_EINVAL


def test_decode_noalloc_uses_the_scratch_and_refuses_what_does_not_fit(lib):
    """kvq_decode_noalloc plans like kvq_decode and puts the partials in the
    library's scratch (the recording launcher's stand-in address); a plan
    whose partials exceed the 64 MiB scratch is refused with ECAPACITY and
    enqueues nothing."""
    h = create(lib, n_seqs=1, n_q_heads=32, n_kv_heads=8, head_dim=128, capacity=9000)
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 8192, None, 0, lib)
    lib.kvq_nodev_clear()
    kvq.kvq_decode(h, Q, kvq.KVQ_BF16, 1, None, 0.1, O, None, WS, 1 << 40, 0, lib)
    with_ws = log(lib)[0]
    lib.kvq_nodev_clear()
    kvq.kvq_decode_noalloc(h, Q, kvq.KVQ_BF16, 1, None, 0.1, O, None, 0, lib)
    assert log(lib) == [with_ws]
    # 512 query rows of 32 heads over 64-row splits: far above 64 MiB of partials
    kvq.kvq_set_split_rows(h, 64, lib)
    need = kvq.kvq_decode_workspace_bytes(h, 512, lib)
    assert need > 64 << 20
    lib.kvq_nodev_clear()
    assert err(lib, kvq.kvq_decode_noalloc, h, Q, kvq.KVQ_BF16, 512, None, 0.1, O, None) == kvq.KVQ_ECAPACITY
    assert log(lib) == [] and "scratch" in kvq.kvq_last_error(lib)
    kvq.kvq_decode(h, Q, kvq.KVQ_BF16, 512, None, 0.1, O, None, WS, 1 << 40, 0, lib)   # the workspace call still works
    assert len(log(lib)) == 1


def test_f8_configuration_rules(lib):
    """K = V = e4m3 rows: 34 bytes per 32 elements for both planes; the stream
    kernel only (head_dim 64, 128 or 256, ring steps on 32-row boundaries),
    so the per-head tiling is refused at decode; mixed formats are refused."""
    s = kvq.kvq_required_bytes(kvq.make_config(2, 8, 2, 128, 100, fmt="e4m3"), lib)
    assert s.k_row_bytes == s.v_row_bytes == 2 * 4 * 34
    assert s.v_planes_bytes == 2 * s.v_session_stride + 256
    E = kvq.KVQ_EUNSUPPORTED
    assert err(lib, kvq.kvq_required_bytes, kvq.make_config(1, 4, 1, 96, 100, fmt="e4m3")) == E
    assert err(lib, kvq.kvq_required_bytes, kvq.make_config(1, 4, 1, 64, 100, 40, 10, fmt="e4m3")) == E
    mixed = kvq.make_config(1, 4, 1, 64, 100)
    mixed.v_fmt = kvq.KVQ_FMT_E4M3
    assert err(lib, kvq.kvq_required_bytes, mixed) == E
    h = create(lib, n_seqs=1, n_q_heads=32, n_kv_heads=8, head_dim=128, capacity=3000, fmt="e4m3")
    kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 2048, None, 0, lib)
    p = plan_of(lib, h)
    assert p["kernel"] == 2
    kvq.kvq_set_decode_tiling(h, kvq.KVQ_DECODE_PER_HEAD, 0, 0, lib)
    lib.kvq_nodev_clear()
    assert err(lib, kvq.kvq_decode, h, Q, kvq.KVQ_BF16, 1, None, 0.1, O, None, WS, 1 << 40) == kvq.KVQ_EINVAL
    assert log(lib) == []
    # an FP8 ring with 32-row steps keeps the stream kernel at every length
    h = create(lib, n_seqs=1, n_q_heads=32, n_kv_heads=8, head_dim=128, capacity=100, window=60,
               ring_step=32, fmt="e4m3")
    for _ in range(120):
        kvq.kvq_append(h, Q, Q, kvq.KVQ_BF16, 1, None, 0, lib)
        assert plan_of(lib, h)["kernel"] == 2
