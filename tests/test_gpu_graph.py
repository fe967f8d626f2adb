"""Steps captured as HIP graphs.  A steady step (append one row per session,
decode, roll the lengths back to where they were) replays to the eager
step's result: on every replay, with eager steps, other work and
synchronisations between the replays; the eager step itself is checked
against the oracle first.  In graph mode one captured step (append, decode)
replays as the lengths grow, each replay against the oracle, and replays
past the plane stop at its capacity."""
import numpy as np
import pytest
import torch

from decode_attention_quantized_append_amd.workloads import round_bf16

pytestmark = pytest.mark.gpu

from gpu_pair import DEV, Pair, assert_close, to_dev  # noqa: E402


def bf16_normal(rng, shape):
    return round_bf16(rng.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("B,H,Hkv,hd,lens", [(1, 32, 8, 128, [8192 - 1]), (3, 40, 8, 128, [700, 1500, 64]),
                                             (2, 16, 4, 256, [900, 333])])
def test_step_graph_replays_equal_eager(B, H, Hkv, hd, lens):
    rng = np.random.default_rng(hd + B)
    p = Pair(B, H, Hkv, hd, max(lens) + 64)
    n = max(lens)
    p.append(bf16_normal(rng, (B, n, Hkv, hd)), bf16_normal(rng, (B, n, Hkv, hd)), lens)
    kn, vn = bf16_normal(rng, (B, 1, Hkv, hd)), bf16_normal(rng, (B, 1, Hkv, hd))
    q = bf16_normal(rng, (B, 1, H, hd))
    scale = hd ** -0.5
    g = p.gpu
    kd, vd, qd = to_dev(kn, "bf16"), to_dev(vn, "bf16"), to_dev(q, "bf16")
    out = torch.empty((B, 1, H, hd), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, 1, H), dtype=torch.float32, device=DEV)
    pre = list(g.host_lengths()[0])

    def step():
        g.append(kd, vd)
        g.decode(qd, scale, out=out, lse=lse)
        g.truncate(pre)

    step()
    torch.cuda.synchronize(DEV)
    want, want_lse = out.clone(), lse.clone()
    p.ref.append(kn, vn)
    ref_o, ref_lse = p.ref.attention(q, scale=scale)
    p.ref.truncate(np.asarray(pre))
    assert_close(want.cpu().numpy(), ref_o, "eager step out")
    assert_close(want_lse.cpu().numpy(), ref_lse, "eager step lse")
    p.check_mirror()

    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(DEV)
    cap.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.graph(graph, stream=cap):
        step()
    torch.cuda.synchronize(DEV)
    filler = torch.empty(1 << 20, dtype=torch.float32, device=DEV)
    for r in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize(DEV)
        assert torch.equal(out, want) and torch.equal(lse, want_lse), f"replay {r} differs from the eager step"
        p.check_mirror()
        filler.normal_()                       # unrelated eager work between replays
        out.zero_()
        step()                                 # and an eager step
        torch.cuda.synchronize(DEV)
        assert torch.equal(out, want), f"eager step after replay {r} differs"


@pytest.mark.parametrize("B,H,Hkv,hd,window,cap,step,pre,steps,fmt",
                         [(2, 32, 8, 128, 0, 700, 0, [500, 77], 24, "q8_0/q5_1"),     # flat: the grid covers the plane
                          (2, 16, 4, 64, 64, 128, 32, [200, 170], 20, "q8_0/q5_1"),  # ring: window + T - 1 + 31 rows
                          (1, 16, 4, 256, 0, 500, 0, [300], 12, "q8_0/q5_1"),
                          (2, 32, 8, 128, 0, 700, 0, [500, 77], 24, "e4m3"),          # FP8 rows, flat and ring
                          (2, 16, 4, 64, 64, 128, 32, [200, 170], 20, "e4m3")])
def test_graph_mode_replays_as_lengths_grow(B, H, Hkv, hd, window, cap, step, pre, steps, fmt):
    """Graph mode: ONE captured step (append a row per session, decode, add
    the attention importance) is replayed `steps` times with no host call
    between replays, each time on the next row and query written into the
    captured input buffers; the device lengths grow by one per replay and
    every replay's output and importance are the oracle's at that length.  Afterwards the host mirror is set from the
    device counters and eager steps continue (through a ring rebase)."""
    rng = np.random.default_rng(hd + cap)
    p = Pair(B, H, Hkv, hd, cap, window, step, fmt=fmt)
    done = np.zeros(B, np.int64)
    while np.any(done < pre):                    # pieces a ring can take without dropping visible rows
        n = np.minimum(np.asarray(pre) - done, 32)
        p.append(bf16_normal(rng, (B, int(n.max()), Hkv, hd)), bf16_normal(rng, (B, int(n.max()), Hkv, hd)),
                 n.tolist())
        done += n
    room = int(min(cap - (p.ref.len - p.ref.base)))
    steps = min(steps, room)                     # replays cannot rebase: stay within the plane
    assert steps >= 5
    g = p.gpu
    g.set_graph_mode(True)
    scale = hd ** -0.5
    kd = torch.zeros((B, 1, Hkv, hd), dtype=torch.bfloat16, device=DEV)
    vd, qd = torch.zeros_like(kd), torch.zeros((B, 1, H, hd), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((B, 1, H, hd), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, 1, H), dtype=torch.float32, device=DEV)
    imp = torch.zeros((B, cap), dtype=torch.float32, device=DEV)
    g.workspace(1)                               # allocated before the capture
    torch.cuda.synchronize(DEV)
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream(DEV)
    cs.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.graph(graph, stream=cs):
        g.append(kd, vd)
        g.decode(qd, scale, out=out, lse=lse)
        g.importance(qd, scale, lse, imp)
    torch.cuda.synchronize(DEV)
    assert g.device_lengths()[0] == pre          # captured, not run
    for r in range(steps):
        kn, vn = bf16_normal(rng, (B, 1, Hkv, hd)), bf16_normal(rng, (B, 1, Hkv, hd))
        q = bf16_normal(rng, (B, 1, H, hd))
        kd.copy_(to_dev(kn, "bf16"))
        vd.copy_(to_dev(vn, "bf16"))
        qd.copy_(to_dev(q, "bf16"))
        out.fill_(float("nan"))
        imp.zero_()
        graph.replay()
        torch.cuda.synchronize(DEV)
        p.ref.append(kn, vn)
        ref_o, ref_lse = p.ref.attention(q, scale=scale)
        assert_close(out.cpu().numpy(), ref_o, f"replay {r} out")
        assert_close(lse.cpu().numpy(), ref_lse, f"replay {r} lse")
        assert_close(imp.cpu().numpy(), p.ref.importance(q, scale=scale), f"replay {r} importance")
    ln, bs, overflow = g.device_lengths()
    assert ln == p.ref.len.tolist() and bs == p.ref.base.tolist() and overflow == 0
    g.set_host_lengths(ln, bs)
    p.check_mirror()
    p.check_planes()
    g.set_graph_mode(False)
    for r in range(3):                           # eager steps from the resynced mirror
        k, v = bf16_normal(rng, (B, 24, Hkv, hd)), bf16_normal(rng, (B, 24, Hkv, hd))
        p.append(k, v)
        p.check_mirror()
        p.decode(bf16_normal(rng, (B, 1, H, hd)), scale, what=f"eager step {r} after replays")
    p.check_planes()


def test_graph_replay_past_the_plane_stops_at_capacity():
    """Replays that would append past the plane: the append kernel drops the
    rows that do not fit, stops len_d at the capacity and sets the overflow
    word; the decode keeps attending to the rows the plane holds."""
    rng = np.random.default_rng(5)
    B, H, Hkv, hd, cap = 2, 8, 2, 128, 300
    pre = [297, 250]
    p = Pair(B, H, Hkv, hd, cap)
    p.append(bf16_normal(rng, (B, 297, Hkv, hd)), bf16_normal(rng, (B, 297, Hkv, hd)), pre)
    g = p.gpu
    g.set_graph_mode(True)
    kd = torch.zeros((B, 1, Hkv, hd), dtype=torch.bfloat16, device=DEV)
    vd, qd = torch.zeros_like(kd), torch.zeros((B, 1, H, hd), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((B, 1, H, hd), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, 1, H), dtype=torch.float32, device=DEV)
    g.workspace(1)
    torch.cuda.synchronize(DEV)
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream(DEV)
    cs.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.graph(graph, stream=cs):
        g.append(kd, vd)
        g.decode(qd, 0.125, out=out, lse=lse)
    torch.cuda.synchronize(DEV)
    for r in range(6):
        kn, vn = bf16_normal(rng, (B, 1, Hkv, hd)), bf16_normal(rng, (B, 1, Hkv, hd))
        q = bf16_normal(rng, (B, 1, H, hd))
        kd.copy_(to_dev(kn, "bf16"))
        vd.copy_(to_dev(vn, "bf16"))
        qd.copy_(to_dev(q, "bf16"))
        graph.replay()
        torch.cuda.synchronize(DEV)
        fits = [int(p.ref.len[b]) < cap for b in range(B)]
        p.ref.append(kn, vn, [1 if f else 0 for f in fits])
        ref_o, ref_lse = p.ref.attention(q, scale=0.125)
        assert_close(out.cpu().numpy(), ref_o, f"replay {r} out")
        ln, bs, overflow = g.device_lengths()
        assert ln == p.ref.len.tolist() and overflow == (1 if r >= 3 else 0)
    assert p.ref.len.tolist() == [300, 256]
    g.set_host_lengths(*g.device_lengths()[:2])
    p.check_mirror()
    p.check_planes()


@pytest.mark.parametrize("fmt", ["q8_0/q5_1", "e4m3"])
def test_graph_mode_verify_rounds_replay(fmt):
    """A speculative-verify round (append 8 drafted rows, decode them
    causally, roll back the 5 not accepted) captured once in graph mode and
    replayed: each replay keeps 3 more rows, and every replay's output is the
    oracle's; q8_0/q5_1 and FP8 rows."""
    rng = np.random.default_rng(77)
    B, H, Hkv, hd, T, keep = 2, 16, 4, 256, 8, 3
    pre = [300, 177]
    p = Pair(B, H, Hkv, hd, 420, fmt=fmt)
    p.append(bf16_normal(rng, (B, 300, Hkv, hd)), bf16_normal(rng, (B, 300, Hkv, hd)), pre)
    g = p.gpu
    g.set_graph_mode(True)
    scale = hd ** -0.5
    kd = torch.zeros((B, T, Hkv, hd), dtype=torch.bfloat16, device=DEV)
    vd, qd = torch.zeros_like(kd), torch.zeros((B, T, H, hd), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((B, T, H, hd), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, T, H), dtype=torch.float32, device=DEV)
    g.workspace(T)
    torch.cuda.synchronize(DEV)
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream(DEV)
    cs.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.graph(graph, stream=cs):
        g.append(kd, vd)
        g.decode(qd, scale, out=out, lse=lse)
        g.rollback([T - keep] * B)
    torch.cuda.synchronize(DEV)
    assert g.device_lengths()[0] == pre
    for r in range(10):
        kn, vn = bf16_normal(rng, (B, T, Hkv, hd)), bf16_normal(rng, (B, T, Hkv, hd))
        q = bf16_normal(rng, (B, T, H, hd))
        kd.copy_(to_dev(kn, "bf16"))
        vd.copy_(to_dev(vn, "bf16"))
        qd.copy_(to_dev(q, "bf16"))
        graph.replay()
        torch.cuda.synchronize(DEV)
        p.ref.append(kn, vn)
        ref_o, ref_lse = p.ref.attention(q, scale=scale)
        p.ref.truncate(p.ref.len - (T - keep))
        assert_close(out.cpu().numpy(), ref_o, f"round {r} out")
        assert_close(lse.cpu().numpy(), ref_lse, f"round {r} lse")
        assert g.device_lengths()[0] == p.ref.len.tolist()
    g.set_host_lengths(*g.device_lengths()[:2])
    p.check_mirror()
    p.check_planes()


def test_rollback_replays_stop_at_the_floor():
    """A captured rollback replayed more often than rows were appended stops
    at the shortest length whose window is resident: 0 in a flat cache, base
    + window in a rebased ring.  Only counters change; no rows are read."""
    rng = np.random.default_rng(9)
    flat = Pair(2, 8, 2, 64, 64)
    flat.append(bf16_normal(rng, (2, 12, 2, 64)), bf16_normal(rng, (2, 12, 2, 64)), [12, 7])
    ring = Pair(1, 8, 2, 64, 48, 16, 16)
    for _ in range(6):
        ring.append(bf16_normal(rng, (1, 10, 2, 64)), bf16_normal(rng, (1, 10, 2, 64)))
    lr, br, _ = ring.gpu.device_lengths()
    assert br[0] > 0
    for p, drop in ((flat, [5, 5]), (ring, [4])):
        graph = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream(DEV)
        cs.wait_stream(torch.cuda.current_stream(DEV))
        with torch.cuda.graph(graph, stream=cs):
            p.gpu.rollback(drop)
        torch.cuda.synchronize(DEV)
        for _ in range(8):
            graph.replay()
        torch.cuda.synchronize(DEV)
    assert flat.gpu.device_lengths()[:2] == ([0, 0], [0, 0])
    ln, bs, _ = ring.gpu.device_lengths()
    assert bs == br and ln == [br[0] + 16]


@pytest.mark.parametrize("window,fmt", [(0, "q8_0/q5_1"), (200, "q8_0/q5_1"), (200, "e4m3")])
def test_graph_mode_prompt_chunks_replay(window, fmt):
    """Prompt chunks in graph mode: ONE captured step (append a chunk of 48
    rows per session, decode all 48 rows causally on the prime kernel, add the
    attention importance) replayed as the lengths grow by 48 per replay, each
    replay's output, lse and importance against the oracle's at that length;
    q8_0/q5_1 and FP8 rows."""
    rng = np.random.default_rng(480 + window)
    B, H, Hkv, hd, T, cap = 2, 16, 4, 128, 48, 1000
    pre = [300, 150]
    p = Pair(B, H, Hkv, hd, cap, window, 0, fmt=fmt)
    p.append(bf16_normal(rng, (B, 300, Hkv, hd)), bf16_normal(rng, (B, 300, Hkv, hd)), pre)
    g = p.gpu
    g.set_graph_mode(True)
    scale = hd ** -0.5
    kd = torch.zeros((B, T, Hkv, hd), dtype=torch.bfloat16, device=DEV)
    vd, qd = torch.zeros_like(kd), torch.zeros((B, T, H, hd), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((B, T, H, hd), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, T, H), dtype=torch.float32, device=DEV)
    imp = torch.zeros((B, cap), dtype=torch.float32, device=DEV)
    g.workspace(T)
    torch.cuda.synchronize(DEV)
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream(DEV)
    cs.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.graph(graph, stream=cs):
        g.append(kd, vd)
        g.decode(qd, scale, out=out, lse=lse)
        g.importance(qd, scale, lse, imp)
    torch.cuda.synchronize(DEV)
    for r in range(8):
        kn, vn = bf16_normal(rng, (B, T, Hkv, hd)), bf16_normal(rng, (B, T, Hkv, hd))
        q = bf16_normal(rng, (B, T, H, hd))
        kd.copy_(to_dev(kn, "bf16"))
        vd.copy_(to_dev(vn, "bf16"))
        qd.copy_(to_dev(q, "bf16"))
        out.fill_(float("nan"))
        imp.zero_()
        graph.replay()
        torch.cuda.synchronize(DEV)
        p.ref.append(kn, vn)
        ref_o, ref_lse = p.ref.attention(q, scale=scale)
        assert_close(out.cpu().numpy(), ref_o, f"replay {r} out")
        assert_close(lse.cpu().numpy(), ref_lse, f"replay {r} lse")
        assert_close(imp.cpu().numpy(), p.ref.importance(q, scale=scale), f"replay {r} importance")
    ln, bs, overflow = g.device_lengths()
    assert ln == p.ref.len.tolist() and bs == p.ref.base.tolist() and overflow == 0
    g.set_host_lengths(ln, bs)
    p.check_mirror()
    p.check_planes()
