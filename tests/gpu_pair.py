"""Drive the HIP path and the oracle side by side on identical inputs.

The inputs are float32 numpy arrays (bf16-representable when the HIP side
takes bf16); the GPU receives them converted exactly, the oracle receives
them as they are.  No value flows from the GPU side to the oracle side.
"""
from __future__ import annotations

import numpy as np
import torch

from decode_attention_quantized_append_amd import KvqLayerCache
from oracle.cache_model import OracleCache

DEV = torch.device("cuda:0")
ATOL, RTOL = 2e-3, 1e-2     # |gpu - oracle| <= ATOL + RTOL * |oracle|, element by element


def to_dev(x: np.ndarray, io: str):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if io == "bf16":
        t = t.to(torch.bfloat16)
        assert torch.equal(t.float(), torch.from_numpy(np.ascontiguousarray(x, np.float32))), "not bf16-exact"
    return t.to(DEV)


def assert_close(got, want, what="", atol=ATOL):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - want)
    bad = err > atol + RTOL * np.abs(want)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + RTOL * np.abs(want))), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu {got[i]!r} oracle {want[i]!r}; max abs err {err.max():.3e}")
    return float(err.max())


class Pair:
    def __init__(self, B, H, Hkv, hd, capacity, window=0, ring_step=0, io="bf16", fmt="q8_0/q5_1"):
        self.B, self.H, self.Hkv, self.hd, self.io, self.fmt = B, H, Hkv, hd, io, fmt
        self.gpu = KvqLayerCache(B, H, Hkv, hd, capacity, window, ring_step, device=DEV, fmt=fmt)
        self.ref = OracleCache(B, Hkv, hd, capacity, window, ring_step, fmt=fmt)
        self.vmax = 0.0

    def append(self, k, v, counts=None):
        self.gpu.append(to_dev(k, self.io), to_dev(v, self.io), counts)
        self.ref.append(k, v, counts)
        self.vmax = max(self.vmax, float(np.abs(v).max()))

    def pv_atol(self):
        """Bound on |o1 - o2| between two GPU decodes of the same rows that
        round P differently to fp16 (other split plans, tilings or row
        groupings).  A decode rounds each weight p to fp16 (relative error at
        most 2^-11), the product with the V step once more (2^-11), and sums
        the rounded weights for the row sum (2^-11): each output is within
        3 * 2^-11 * max |v| of the fp32 result, so two are within
        3 * 2^-10 * max |v|.  max |v| is taken from the appended rows, with
        5 % for the q5_1 rounding of the codes."""
        return 3 * 2.0 ** -10 * 1.05 * self.vmax

    def lse_atol(self):
        """Bound on |lse1 - lse2| between two such decodes: each row sum adds
        weights rounded to fp16, within a factor 1 +- 2^-11 of the exact sum,
        so each log-sum-exp is within log(1 + 2^-11) < 4.9e-4 of it."""
        return 2 * 4.9e-4

    def truncate(self, new_len):
        self.gpu.truncate(list(new_len))
        self.ref.truncate(np.asarray(new_len))

    def check_mirror(self):
        ln, bs = self.gpu.host_lengths()
        assert ln == self.ref.len.tolist() and bs == self.ref.base.tolist()
        dev = self.gpu.counters[:2 * self.B].cpu().numpy()
        assert dev[:self.B].tolist() == ln and dev[self.B:].tolist() == bs, "device counters out of step"

    def check_planes(self, rows=None):
        """Live physical rows of every session, byte for byte (all of them, or
        the physical row indices in `rows`)."""
        kp, vp = self.gpu.planes()
        for b in range(self.B):
            n = int(self.ref.len[b] - self.ref.base[b])
            sel = np.arange(n) if rows is None else np.asarray([r for r in rows if r < n], dtype=np.int64)
            if sel.size == 0:
                continue
            idx = torch.from_numpy(sel).to(DEV)
            gk = kp[b].index_select(0, idx).cpu().numpy()
            gv = vp[b].index_select(0, idx).cpu().numpy()
            rk, rv = self.ref.k[b][sel], self.ref.v[b][sel]
            vb = 34 if self.fmt == "e4m3" else 24     # an FP8 row shows as 34-byte groups
            for name, g, r, bb in (("K", gk, rk, 34), ("V", gv, rv, vb)):
                if not np.array_equal(g, r):
                    i = np.nonzero((g != r).any(1))[0][0]
                    gb, rb = g[i].reshape(-1, bb), r[i].reshape(-1, bb)
                    blks = np.nonzero((gb != rb).any(1))[0]
                    j = blks[0]
                    raise AssertionError(
                        f"{name} bytes differ: session {b}, physical row {sel[i]}, blocks {blks.tolist()}; "
                        f"block {j}: gpu {bytes(gb[j]).hex(' ')} oracle {bytes(rb[j]).hex(' ')}")

    def decode(self, q, scale, sinks=None, sel=None, what="decode", atol=ATOL):
        T = q.shape[1]
        s_dev = torch.from_numpy(sinks).to(DEV) if sinks is not None else None
        out, lse = self.gpu.decode(to_dev(q, self.io), scale, sinks=s_dev)
        torch.cuda.synchronize(DEV)
        want, want_lse = self.ref.attention(q, scale=scale, sinks=sinks, sel=sel)
        got, got_lse = out.cpu().numpy(), lse.cpu().numpy()
        if sel is not None:
            flat = np.asarray(sel)
            got = got.reshape(-1, self.hd)[flat]
            want = want.reshape(-1, self.hd)[flat]
            got_lse, want_lse = got_lse.reshape(-1)[flat], want_lse.reshape(-1)[flat]
        e = assert_close(got, want, what + " out", atol)
        assert_close(got_lse, want_lse, what + " lse")
        assert T == q.shape[1]
        return e
