"""Cache model of the oracle: physical K/V planes per session, the committed
length ``len`` and the ring base ``base``.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Written from the memra-engine pages:
* "Struct KvLayer", fields len_d / base_d: the live view of a session is the
  logical rows [max(0, len - window), len); a logical row lives at physical
  row ``row - base``; only a rebase moves ``base``; rewinds move ``len`` only.
* "Struct KvLayer", field ring: ``len`` stays absolute; no ring means the flat
  addressing [0, capacity).
* "Struct Cache", method rollback: rolling back sets ``len`` (no copy).
Readings where the pages are silent:
* a rebase happens when an append would write past the last physical row; it
  advances ``base`` by whole ``ring_step`` units until the append fits and
  moves the surviving rows [new_base, len) down to physical row 0;
* an append may not drop a row that its first new row can still see:
  max(0, len + 1 - window) >= new_base, else RangeError;
* truncate only shrinks, and in a windowed ring keeps
  max(0, new_len - window) >= base, else RangeError.
"""
from __future__ import annotations

import numpy as np

from . import core


class RangeError(ValueError):
    """A logical row the call needs is not resident (ring rebased past it)."""


class CapacityError(ValueError):
    """A flat cache has no physical row left for the append."""


class OracleCache:
    """fmt: "q8_0/q5_1" (K q8_0, V q5_1) or "e4m3" (K and V FP8 rows: the
    codes of a row's blocks, then their fp16 scales; see kvq_oracle.c)."""

    def __init__(self, n_seqs, n_kv_heads, head_dim, capacity, window=0, ring_step=0, fmt="q8_0/q5_1"):
        if head_dim % 32 != 0:
            raise ValueError("head_dim must be a multiple of 32 (a block never straddles a head)")
        self.fmt = core.FORMATS[fmt]
        if ring_step and (window <= 0 or window + ring_step > capacity):
            raise ValueError("a ring needs 0 < window and window + ring_step <= capacity")
        self.B, self.Hkv, self.hd = int(n_seqs), int(n_kv_heads), int(head_dim)
        self.cap, self.window, self.step = int(capacity), int(window), int(ring_step)
        nb = self.Hkv * self.hd // 32
        self.k_row, self.v_row = nb * 34, nb * (34 if self.fmt == core.FMT_E4M3 else 24)
        self.k = np.zeros((self.B, self.cap, self.k_row), dtype=np.uint8)
        self.v = np.zeros((self.B, self.cap, self.v_row), dtype=np.uint8)
        self.len = np.zeros(self.B, dtype=np.int64)
        self.base = np.zeros(self.B, dtype=np.int64)

    # -- planning (no state change) ------------------------------------
    def plan_base(self, b: int, n: int) -> int:
        """The base session b must have before appending n rows."""
        L, base = int(self.len[b]), int(self.base[b])
        if n == 0:
            return base
        if not self.step:
            if L + n > self.cap:
                raise CapacityError(f"session {b}: {L}+{n} rows exceed capacity {self.cap}")
            return base
        while L + n - base > self.cap:
            base += self.step
        if base != int(self.base[b]) and max(0, L + 1 - self.window) < base:
            raise RangeError(f"session {b}: rebase to {base} would drop visible rows")
        return base

    # -- state changes ---------------------------------------------------
    def append(self, k, v, counts=None):
        """k, v: float32 [B, T, Hkv, hd].  Session b appends its first
        counts[b] rows (all T when counts is None)."""
        k = np.asarray(k, dtype=np.float32)
        v = np.asarray(v, dtype=np.float32)
        B, T, Hkv, hd = k.shape
        assert (B, Hkv, hd) == (self.B, self.Hkv, self.hd) and v.shape == k.shape
        counts = np.full(B, T, dtype=np.int64) if counts is None else np.asarray(counts, np.int64)
        if np.any(counts < 0) or np.any(counts > T):
            raise ValueError("counts out of [0, T]")
        new_base = [self.plan_base(b, int(counts[b])) for b in range(B)]   # refuse before changing
        for b in range(B):
            n, L, old = int(counts[b]), int(self.len[b]), int(self.base[b])
            if n == 0:
                continue
            nb_ = new_base[b]
            if nb_ != old:   # move the surviving rows [nb_, L) to physical 0
                keep = L - nb_
                self.k[b, :keep] = self.k[b, nb_ - old: L - old].copy()
                self.v[b, :keep] = self.v[b, nb_ - old: L - old].copy()
                self.base[b] = nb_
            p0 = L - nb_
            if self.fmt == core.FMT_E4M3:
                self.k[b, p0:p0 + n] = core.quantize_f8_rows(k[b, :n], Hkv * hd).reshape(n, self.k_row)
                self.v[b, p0:p0 + n] = core.quantize_f8_rows(v[b, :n], Hkv * hd).reshape(n, self.v_row)
            else:
                self.k[b, p0:p0 + n] = core.quantize_k(k[b, :n]).reshape(n, self.k_row)
                self.v[b, p0:p0 + n] = core.quantize_v(v[b, :n]).reshape(n, self.v_row)
            self.len[b] = L + n

    def truncate(self, new_len):
        new_len = np.asarray(new_len, dtype=np.int64)
        if np.any(new_len < 0) or np.any(new_len > self.len):
            raise ValueError("truncate only shrinks")
        if self.step:
            lo = np.maximum(0, new_len - self.window)
            if np.any(lo < self.base):
                raise RangeError("truncate would expose rows the ring no longer holds")
        self.len = new_len.copy()

    # -- reading -----------------------------------------------------------
    def live_rows(self, b: int):
        """(first logical row held, len): physical rows [0, len - base)."""
        return int(self.base[b]), int(self.len[b])

    def importance(self, q, *, scale, sinks=None):
        """float64 [B, capacity]: probability mass per physical row, summed
        over the T query rows (the last T rows) and the H heads of q."""
        q = np.asarray(q, dtype=np.float32)
        B, T, H, hd = q.shape
        if np.any(self.len < T):
            raise ValueError("each session needs at least T committed rows")
        return core.importance(q, [self.k[b] for b in range(B)], self.base, self.len, self.cap,
                               n_kv_heads=self.Hkv, window=self.window, sinks=sinks, scale=scale,
                               fmt=self.fmt)

    def attention(self, q, *, scale, sinks=None, sel=None, want_lse=True):
        """q: float32 [B, T, H, hd]; the T query rows are the last T rows."""
        q = np.asarray(q, dtype=np.float32)
        B, T, H, hd = q.shape
        if np.any(self.len < T):
            raise ValueError("each session needs at least T committed rows")
        if self.window:
            lo = np.maximum(0, self.len - T + 1 - self.window)
            if np.any(lo < self.base):
                raise RangeError("visible rows are no longer resident")
        elif np.any(self.base != 0):
            raise RangeError("full attention over a rebased ring")
        return core.attention(q, [self.k[b] for b in range(B)], [self.v[b] for b in range(B)],
                              self.base, self.len, n_kv_heads=self.Hkv, window=self.window,
                              sinks=sinks, scale=scale, sel=sel, want_lse=want_lse, fmt=self.fmt)
