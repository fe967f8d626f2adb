"""A decode step captured as one HIP graph (append one row per session,
decode, roll the lengths back to where they were) replays to the eager
step's result: on every replay, with eager steps, other work and
synchronisations between the replays.  The eager step itself is checked
against the oracle first."""
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
