"""kvq_decode_noalloc (the decode whose split-K partials live in the
library's own device scratch instead of a caller workspace) through the C
ABI, against kvq_decode on the same inputs: two calls in a row on one
device, the second with a smaller input, each equal to kvq_decode's result
(the same kernels and plan, so bit for bit) and within the oracle's
tolerance."""
import numpy as np
import pytest
import torch

from decode_attention_quantized_append_amd import kvq
from decode_attention_quantized_append_amd.workloads import round_bf16

pytestmark = pytest.mark.gpu

from gpu_pair import DEV, Pair, assert_close, to_dev  # noqa: E402


def filled(rng, B, H, Hkv, hd, lens, io, fmt="q8_0/q5_1"):
    p = Pair(B, H, Hkv, hd, max(lens) + 16, io=io, fmt=fmt)
    lens = np.asarray(lens)
    done = np.zeros(B, np.int64)
    while np.any(done < lens):
        n = np.minimum(lens - done, 500)
        m = int(n.max())
        k = rng.standard_normal((B, m, Hkv, hd)).astype(np.float32)
        v = rng.standard_normal((B, m, Hkv, hd)).astype(np.float32)
        if io == "bf16":
            k, v = round_bf16(k), round_bf16(v)
        p.append(k, v, n.tolist())
        done += n
    return p


def both(p, rng, T, io, sinks=False):
    q = rng.standard_normal((p.B, T, p.H, p.hd)).astype(np.float32)
    q = round_bf16(q) if io == "bf16" else q
    s = rng.standard_normal(p.H).astype(np.float32) if sinks else None
    scale = float(np.float32(1 / np.sqrt(p.hd)))
    qd = to_dev(q, io)
    sd = torch.from_numpy(s).to(DEV) if s is not None else None
    out_ws, lse_ws = p.gpu.decode(qd, scale, sinks=sd)                  # kvq_decode, torch workspace
    out = torch.full_like(out_ws, float("nan"))
    lse = torch.full_like(lse_ws, float("nan"))
    kvq.kvq_decode_noalloc(p.gpu.h, qd.data_ptr(), p.gpu._dtype(qd), T, sd.data_ptr() if sd is not None else None,
                           scale, out.data_ptr(), lse.data_ptr(), p.gpu._stream(), p.gpu.lib)
    torch.cuda.synchronize(DEV)
    assert torch.equal(out, out_ws) and torch.equal(lse, lse_ws), "noalloc differs from kvq_decode"
    want, want_lse = p.ref.attention(q, scale=scale, sinks=s)
    assert_close(out.cpu().numpy(), want, "noalloc out")
    assert_close(lse.cpu().numpy(), want_lse, "noalloc lse")


def test_noalloc_equals_decode_two_calls_second_smaller():
    rng = np.random.default_rng(77)
    # a verify-like call (256-dim heads, 8 causal rows, two sessions) ...
    big = filled(rng, 2, 16, 4, 256, [3000, 1700], "bf16")
    both(big, rng, 8, "bf16", sinks=True)
    # ... then a smaller one on the same device: fewer sessions, rows, heads and
    # query rows, so that the scratch still holds the first call's partials
    small = filled(rng, 1, 8, 2, 128, [300], "f32")
    both(small, rng, 1, "f32")
    # and the first handle again
    both(big, rng, 2, "bf16")


def test_noalloc_prompt_chunk_and_fp8_rows():
    """FP8 rows: a prompt chunk of 64 rows (eight groups of query rows, the
    prime kernel), then a smaller verify-like call on another handle, each
    equal to kvq_decode bit for bit."""
    rng = np.random.default_rng(79)
    chunk = filled(rng, 1, 32, 8, 128, [900], "bf16", fmt="e4m3")
    both(chunk, rng, 64, "bf16", sinks=True)
    small = filled(rng, 2, 16, 4, 256, [400, 200], "bf16", fmt="e4m3")
    both(small, rng, 8, "bf16")


def test_noalloc_refuses_partials_beyond_the_scratch():
    rng = np.random.default_rng(78)
    p = filled(rng, 1, 32, 8, 128, [4096], "bf16")
    p.gpu.set_split_rows(64)
    assert kvq.kvq_decode_workspace_bytes(p.gpu.h, 512, p.gpu.lib) > 64 << 20
    q = to_dev(round_bf16(rng.standard_normal((1, 512, 32, 128)).astype(np.float32)), "bf16")
    out = torch.empty((1, 512, 32, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_noalloc(p.gpu.h, q.data_ptr(), kvq.KVQ_BF16, 512, None, 0.1, out.data_ptr(), None,
                               p.gpu._stream(), p.gpu.lib)
    assert e.value.status == kvq.KVQ_ECAPACITY
