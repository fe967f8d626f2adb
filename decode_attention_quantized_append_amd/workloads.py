"""Seeded synthetic workloads: shapes, lengths and input tensors.

This module holds generators only -- no quantization, no attention, nothing
of the method's arithmetic -- so that both the HIP path and the CPU oracle
can be fed from it without sharing any of the computation.

Every random array is drawn from a counter-keyed stream: ``numpy``'s
``SeedSequence`` keyed by (workload seed, stream id, session, chunk), so any
chunk of rows can be regenerated on its own, in any order.  bf16 inputs are
the float32 draws rounded to bfloat16 (round to nearest even); the float32
arrays returned here always hold exactly the values the GPU receives.

Workloads (one attention layer each):
  tiny      1 session, 4 Q / 1 KV heads, head_dim 64, 256 cached rows, T=1,
            fp32 q/k/v ~ N(0,1)
  qwen_gqa  1 session, 32 Q / 8 KV heads, head_dim 128, 8192 cached rows, T=1,
            bf16 q ~ N(0,1); k ~ N(0,1) with 4 outlier channels per KV head
            scaled x8; v ~ N(0, 0.5^2)
  batched   16 sessions, cached rows uniform on [1024, 32768], 40 Q / 8 KV
            heads, head_dim 128, T=1, bf16, k/v ~ N(0,1)
  sink_ring 4 sessions, 64 Q / 8 KV heads, head_dim 64, window 1024 served
            from a 2048-row ring advancing 512 rows at a time, absolute length
            131072, sinks ~ N(0,1) fp32, bf16 q/k/v ~ N(0,1)
  verify    2 sessions, 16 Q / 4 KV heads, head_dim 256, 131072 cached rows,
            T=8 causal verify rows, then rollback to len+3, bf16 q/k/v ~ N(0,1)
  prime     a prompt chunk: 1 session of the qwen_gqa shape and inputs, 512
            rows appended and attending causally, each within a 4096-row
            sliding window, at 32768 rows, served from a 5118-row ring that
            advances 512 rows at a time (not one of the five measured
            configurations: the chunked prime of a long prompt)
  verify_f8, batched_f8, prime_f8
            the verify, batched and prime inputs (the same seeds) held as
            FP8 (e4m3) K and V rows
The k/v distribution named "as config 1" for the batched and verify shapes
is read as the tiny shape's N(0,1); ``kv_dist="outlier"`` selects the other
reading (the qwen_gqa distribution).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

CHUNK = 1024          # rows per generator chunk
_Q, _K, _V, _SINK, _OUTL, _LEN = 1, 2, 3, 4, 5, 6


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values that are exactly bf16 -> their uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value is not a bfloat16"
    return (u >> 16).astype(np.uint16)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    H: int
    Hkv: int
    hd: int
    T: int
    cached: int                      # rows the last query row sees (fixed-length shapes)
    ragged: Optional[tuple] = None   # (lo, hi) inclusive per-session lengths
    window: int = 0
    ring_cap: int = 0                # physical rows of the ring (0 = flat)
    ring_step: int = 0
    sinks: bool = False
    io_dtype: str = "bf16"           # q/k/v input dtype: "f32" or "bf16"
    kv_dist: str = "normal"          # "normal" | "outlier" (outlier channels, v std 0.5)
    rollback_keep: int = 0           # after a T-row verify, keep this many of the T rows
    fmt: str = "q8_0/q5_1"           # cache format: "q8_0/q5_1" or "e4m3" (K and V FP8 rows)

    @property
    def hpk(self) -> int:
        return self.H // self.Hkv

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.hd)))

    @property
    def k_row_bytes(self) -> int:
        return self.Hkv * self.hd // 32 * 34

    @property
    def v_row_bytes(self) -> int:
        return self.Hkv * self.hd // 32 * (34 if self.fmt == "e4m3" else 24)

    def lengths(self) -> np.ndarray:
        """Committed rows per session after the step's append (the last query
        row sees exactly this many rows, before any window)."""
        if self.ragged:
            lo, hi = self.ragged
            return _rng(self.seed, _LEN).integers(lo, hi + 1, size=self.B).astype(np.int64)
        return np.full(self.B, self.cached, dtype=np.int64)

    def visible(self) -> np.ndarray:
        n = self.lengths()
        return np.minimum(n, self.window) if self.window else n

    def capacity(self, extra_steps: int = 0) -> int:
        if self.ring_cap:
            return self.ring_cap
        grow = max(self.T, self.rollback_keep * max(extra_steps, 1) + self.T)
        return int(self.lengths().max()) + grow + 64

    def span(self) -> np.ndarray:
        """Rows per session that the step's T query rows see together: the
        last row's visible rows and, with a window, the T - 1 rows below."""
        n = self.lengths()
        return np.minimum(n, self.window + self.T - 1) if self.window else n

    def attn_flops_per_decode(self) -> int:
        """Multiply-adds x 2 of the attention the T query rows make: for each
        query row and Q head, q.k and p.v over the rows it sees."""
        n = self.lengths()
        total = 0
        for t in range(self.T):
            upto = n - self.T + t + 1
            vis = np.minimum(upto, self.window) if self.window else upto
            total += int(vis.sum())
        return 4 * self.hd * self.H * total

    def kv_bytes_per_decode(self) -> int:
        """Algorithmic K+V bytes one decode reads: the rows its query rows
        see (each once) x row bytes."""
        return int(self.span().sum()) * (self.k_row_bytes + self.v_row_bytes)

    # -- generators ------------------------------------------------------
    def _cast(self, x: np.ndarray) -> np.ndarray:
        return round_bf16(x) if self.io_dtype == "bf16" else x.astype(np.float32)

    def outlier_channels(self) -> np.ndarray:
        """[Hkv, 4] distinct channel indices per KV head, fixed for the run."""
        g = _rng(self.seed, _OUTL)
        return np.stack([g.choice(self.hd, size=4, replace=False) for _ in range(self.Hkv)])

    def kv_rows(self, b: int, r0: int, r1: int):
        """(k, v) float32 [r1-r0, Hkv, hd] for logical rows [r0, r1) of session b."""
        ks, vs = [], []
        c0, c1 = r0 // CHUNK, (r1 - 1) // CHUNK if r1 > r0 else r0 // CHUNK - 1
        for c in range(c0, c1 + 1):
            shape = (CHUNK, self.Hkv, self.hd)
            k = _rng(self.seed, _K, b, c).standard_normal(shape, dtype=np.float32)
            v = _rng(self.seed, _V, b, c).standard_normal(shape, dtype=np.float32)
            if self.kv_dist == "outlier":
                oc = self.outlier_channels()
                for g in range(self.Hkv):
                    k[:, g, oc[g]] *= 8.0
                v *= 0.5
            lo, hi = max(r0, c * CHUNK) - c * CHUNK, min(r1, (c + 1) * CHUNK) - c * CHUNK
            ks.append(k[lo:hi])
            vs.append(v[lo:hi])
        if not ks:
            e = np.zeros((0, self.Hkv, self.hd), np.float32)
            return e, e.copy()
        return self._cast(np.concatenate(ks)), self._cast(np.concatenate(vs))

    def kv_block(self, rows_per_session, start_rows, T: int):
        """(k, v) float32 [B, T, Hkv, hd]: session b's rows
        [start_rows[b], start_rows[b] + rows_per_session[b]) in its first slots,
        zeros after."""
        k = np.zeros((self.B, T, self.Hkv, self.hd), np.float32)
        v = np.zeros_like(k)
        for b in range(self.B):
            n, s = int(rows_per_session[b]), int(start_rows[b])
            if n:
                k[b, :n], v[b, :n] = self.kv_rows(b, s, s + n)
        return k, v

    def pre_step_lengths(self) -> np.ndarray:
        """Committed rows per session before a step appends its T rows."""
        return self.lengths() - self.T

    def prefill_pieces(self, piece: int = 1024):
        """Setup appends that bring an empty cache to ``pre_step_lengths()``:
        yields (rows per session, first logical row per session, T) for each
        append call.  A ring gets pieces no longer than capacity - window -
        ring_step + 2 rows, so that no rebase can drop a visible row."""
        target = self.pre_step_lengths()
        if self.ring_cap:
            piece = min(piece, self.ring_cap - self.window - self.ring_step + 2)
        done = np.zeros(self.B, dtype=np.int64)
        while np.any(done < target):
            n = np.minimum(target - done, piece)
            yield n.copy(), done.copy(), int(n.max())
            done += n

    def q(self, step: int = 0) -> np.ndarray:
        """float32 [B, T, H, hd] query rows of decode step ``step``."""
        g = _rng(self.seed, _Q, step)
        return self._cast(g.standard_normal((self.B, self.T, self.H, self.hd), dtype=np.float32))

    def sink_logits(self) -> Optional[np.ndarray]:
        if not self.sinks:
            return None
        return _rng(self.seed, _SINK).standard_normal(self.H, dtype=np.float32)


WORKLOADS = {
    "tiny": Workload("tiny", 101, B=1, H=4, Hkv=1, hd=64, T=1, cached=256, io_dtype="f32"),
    "qwen_gqa": Workload("qwen_gqa", 102, B=1, H=32, Hkv=8, hd=128, T=1, cached=8192,
                         kv_dist="outlier"),
    "batched": Workload("batched", 103, B=16, H=40, Hkv=8, hd=128, T=1, cached=0,
                        ragged=(1024, 32768)),
    "sink_ring": Workload("sink_ring", 104, B=4, H=64, Hkv=8, hd=64, T=1, cached=131072,
                          window=1024, ring_cap=2048, ring_step=512, sinks=True),
    "verify": Workload("verify", 105, B=2, H=16, Hkv=4, hd=256, T=8, cached=131072,
                       rollback_keep=3),
    # the prompt chunk is served from a ring of the rows kvq_ring_rows gives
    # for a 4096-row window, 512-row chunks and 512-row steps
    "prime": Workload("prime", 106, B=1, H=32, Hkv=8, hd=128, T=512, cached=32768,
                      window=4096, ring_cap=4096 + 512 + 512 - 2, ring_step=512, kv_dist="outlier"),
    # the FP8 (e4m3) K/V variant on the two long-context shapes: the same
    # seeds, so the same inputs, held as FP8 rows
    "verify_f8": Workload("verify_f8", 105, B=2, H=16, Hkv=4, hd=256, T=8, cached=131072,
                          rollback_keep=3, fmt="e4m3"),
    "batched_f8": Workload("batched_f8", 103, B=16, H=40, Hkv=8, hd=128, T=1, cached=0,
                           ragged=(1024, 32768), fmt="e4m3"),
    "prime_f8": Workload("prime_f8", 106, B=1, H=32, Hkv=8, hd=128, T=512, cached=32768,
                         window=4096, ring_cap=4096 + 512 + 512 - 2, ring_step=512, kv_dist="outlier",
                         fmt="e4m3"),
}


def get(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return dataclasses.replace(w, **overrides) if overrides else w
