"""ctypes wrapper of the plain C oracle (``kvq_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).  The wrapper marshals
arrays; every step of the arithmetic is in the C file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

GCC_FLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11"]


def build_oracle(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (no fast-math: IEEE division and rintf)."""
    cmd = ["gcc", *GCC_FLAGS, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str | None = None):
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    # KVQ_ORACLE_LIB: another build of the same source (the sanitizer test's)
    p = path or os.environ.get("KVQ_ORACLE_LIB") or _LIB
    if not os.path.exists(p):
        build_oracle(out=p)
    lib = ctypes.CDLL(p)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    lib.kvqo_f32_to_f16.argtypes = [ctypes.c_float]
    lib.kvqo_f32_to_f16.restype = ctypes.c_uint16
    lib.kvqo_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.kvqo_f16_to_f32.restype = ctypes.c_float
    lib.kvqo_f32_to_f16_array.argtypes = [f32p, u16p, ctypes.c_int64]
    for name in ("kvqo_q8_0_encode", "kvqo_q5_1_encode"):
        getattr(lib, name).argtypes = [f32p, u8p]
    for name in ("kvqo_q8_0_decode", "kvqo_q5_1_decode"):
        getattr(lib, name).argtypes = [u8p, f64p]
    lib.kvqo_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.kvqo_e4m3_value.restype = ctypes.c_double
    lib.kvqo_e4m3_from_f32.argtypes = [ctypes.c_float]
    lib.kvqo_e4m3_from_f32.restype = ctypes.c_uint8
    lib.kvqo_f8_encode.argtypes = [f32p, u8p]
    lib.kvqo_f8_decode.argtypes = [u8p, f64p]
    for name in ("kvqo_quantize_k", "kvqo_quantize_v"):
        getattr(lib, name).argtypes = [f32p, ctypes.c_int64, u8p]
    lib.kvqo_quantize_f8_rows.argtypes = [f32p, ctypes.c_int64, ctypes.c_int32, u8p]
    lib.kvqo_attention.argtypes = [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        f32p, ctypes.POINTER(u8p), ctypes.POINTER(u8p), i64p, i64p, ctypes.c_int32,
        f32p, ctypes.c_float, i64p, ctypes.c_int64, f32p, f32p]
    lib.kvqo_attention.restype = ctypes.c_int
    lib.kvqo_importance.argtypes = [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        f32p, ctypes.POINTER(u8p), i64p, i64p, ctypes.c_int32, f32p, ctypes.c_float, f64p, ctypes.c_int64]
    lib.kvqo_importance.restype = ctypes.c_int
    lib.kvqo_max_threads.restype = ctypes.c_int
    lib.kvqo_set_threads.argtypes = [ctypes.c_int]
    lib.kvqo_set_threads.restype = None
    if path is None:
        _lib = lib
    return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the float32 values they denote (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_f16(x, lib=None) -> np.ndarray:
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(x.shape, dtype=np.uint16)
    lib.kvqo_f32_to_f16_array(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint16), x.size)
    return out


def f16_to_f32(h, lib=None) -> np.ndarray:
    lib = lib or load()
    h = np.asarray(h, dtype=np.uint16).ravel()
    return np.array([lib.kvqo_f16_to_f32(int(v)) for v in h], dtype=np.float32)


def _block_op(fn, x, in_dtype, in_size, out_dtype, out_size):
    x = np.ascontiguousarray(x, dtype=in_dtype)
    assert x.size == in_size
    out = np.empty(out_size, dtype=out_dtype)
    in_c = ctypes.c_float if in_dtype == np.float32 else ctypes.c_uint8
    out_c = ctypes.c_uint8 if out_dtype == np.uint8 else ctypes.c_double
    fn(_ptr(x, in_c), _ptr(out, out_c))
    return out


def q8_0_encode(x, lib=None):
    return _block_op((lib or load()).kvqo_q8_0_encode, x, np.float32, 32, np.uint8, 34)


def q8_0_decode(b, lib=None):
    return _block_op((lib or load()).kvqo_q8_0_decode, b, np.uint8, 34, np.float64, 32)


def q5_1_encode(x, lib=None):
    return _block_op((lib or load()).kvqo_q5_1_encode, x, np.float32, 32, np.uint8, 24)


def q5_1_decode(b, lib=None):
    return _block_op((lib or load()).kvqo_q5_1_decode, b, np.uint8, 24, np.float64, 32)


def e4m3_value(codes, lib=None) -> np.ndarray:
    """Value of each e4m3 code (OCP FP8 E4M3; NaN for S.1111.111), float64."""
    lib = lib or load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.kvqo_e4m3_value(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


def e4m3_from_f32(x, lib=None) -> np.ndarray:
    """Nearest e4m3 code of each float32 (ties to even, saturating at +-448)."""
    lib = lib or load()
    a = np.asarray(x, dtype=np.float32)
    return np.array([lib.kvqo_e4m3_from_f32(float(v)) for v in a.ravel()], dtype=np.uint8).reshape(a.shape)


def f8_encode(x, lib=None):
    """32 float32 values per block -> 34-byte FP8 blocks (fp16 scale + 32 e4m3 codes)."""
    return _block_op((lib or load()).kvqo_f8_encode, x, np.float32, 32, np.uint8, 34)


def f8_decode(b, lib=None):
    return _block_op((lib or load()).kvqo_f8_decode, b, np.uint8, 34, np.float64, 32)


def _quantize(fn, x, blk_bytes):
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.size % 32 == 0
    out = np.empty(x.size // 32 * blk_bytes, dtype=np.uint8)
    fn(_ptr(x, ctypes.c_float), x.size, _ptr(out, ctypes.c_uint8))
    return out


def quantize_k(x, lib=None) -> np.ndarray:
    """float32 values (any shape, size % 32 == 0) -> q8_0 bytes, flat."""
    return _quantize((lib or load()).kvqo_quantize_k, x, 34)


def quantize_v(x, lib=None) -> np.ndarray:
    """float32 values (any shape, size % 32 == 0) -> q5_1 bytes, flat."""
    return _quantize((lib or load()).kvqo_quantize_v, x, 24)


# cache formats (kvq_oracle.h KVQO_FMT_*)
FMT_Q8_Q5, FMT_E4M3 = 0, 1
FORMATS = {"q8_0/q5_1": FMT_Q8_Q5, "e4m3": FMT_E4M3}


def quantize_f8_rows(x, row_elems, lib=None) -> np.ndarray:
    """float32 values, rows of row_elems (a multiple of 32) -> FP8 row bytes,
    flat: per row the codes of its blocks, then their fp16 scales."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.size % row_elems == 0 and row_elems % 32 == 0
    n_rows = x.size // row_elems
    out = np.empty(n_rows * row_elems // 32 * 34, dtype=np.uint8)
    lib.kvqo_quantize_f8_rows(_ptr(x, ctypes.c_float), n_rows, int(row_elems), _ptr(out, ctypes.c_uint8))
    return out


def attention(q, k_planes, v_planes, base, length, *, n_kv_heads, window=0,
              sinks=None, scale, sel=None, want_lse=True, fmt=FMT_Q8_Q5, lib=None):
    """Exact attention.  q: float32 [B, T, H, hd].  k_planes / v_planes: per
    session uint8 arrays whose row 0 holds logical row base[b], in cache
    format fmt.  Returns (out [B,T,H,hd] float32, lse [B,T,H] float32 or
    None); entries not in ``sel`` are NaN."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, T, H, hd = q.shape
    u8p = ctypes.POINTER(ctypes.c_uint8)
    kp = [np.ascontiguousarray(p, dtype=np.uint8) for p in k_planes]
    vp = [np.ascontiguousarray(p, dtype=np.uint8) for p in v_planes]
    karr = (u8p * B)(*[_ptr(p, ctypes.c_uint8) for p in kp])
    varr = (u8p * B)(*[_ptr(p, ctypes.c_uint8) for p in vp])
    base = np.ascontiguousarray(base, dtype=np.int64)
    length = np.ascontiguousarray(length, dtype=np.int64)
    out = np.full((B, T, H, hd), np.nan, dtype=np.float32)
    lse = np.full((B, T, H), np.nan, dtype=np.float32) if want_lse else None
    s = None
    if sinks is not None:
        s = np.ascontiguousarray(sinks, dtype=np.float32)
        assert s.shape == (H,)
    selarr = None
    if sel is not None:
        selarr = np.ascontiguousarray(sel, dtype=np.int64)
    rc = lib.kvqo_attention(
        int(fmt), B, T, H, int(n_kv_heads), hd, _ptr(q, ctypes.c_float), karr, varr,
        _ptr(base, ctypes.c_int64), _ptr(length, ctypes.c_int64), int(window),
        _ptr(s, ctypes.c_float) if s is not None else None, float(scale),
        _ptr(selarr, ctypes.c_int64) if selarr is not None else None,
        0 if selarr is None else selarr.size,
        _ptr(out, ctypes.c_float), _ptr(lse, ctypes.c_float) if lse is not None else None)
    if rc != 0:
        raise ValueError("oracle attention: argument outside the method's domain")
    return out, lse


def importance(q, k_planes, base, length, capacity, *, n_kv_heads, window=0, sinks=None, scale,
               fmt=FMT_Q8_Q5, lib=None):
    """Attention importance: float64 [B, capacity], the probability mass of
    each physical row summed over the T query rows and H heads of q (float32
    [B, T, H, hd], the last T rows); rows no query row sees stay 0."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, T, H, hd = q.shape
    u8p = ctypes.POINTER(ctypes.c_uint8)
    kp = [np.ascontiguousarray(p, dtype=np.uint8) for p in k_planes]
    karr = (u8p * B)(*[_ptr(p, ctypes.c_uint8) for p in kp])
    base = np.ascontiguousarray(base, dtype=np.int64)
    length = np.ascontiguousarray(length, dtype=np.int64)
    s = None
    if sinks is not None:
        s = np.ascontiguousarray(sinks, dtype=np.float32)
        assert s.shape == (H,)
    imp = np.zeros((B, int(capacity)), dtype=np.float64)
    rc = lib.kvqo_importance(int(fmt), B, T, H, int(n_kv_heads), hd, _ptr(q, ctypes.c_float), karr,
                             _ptr(base, ctypes.c_int64), _ptr(length, ctypes.c_int64), int(window),
                             _ptr(s, ctypes.c_float) if s is not None else None, float(scale),
                             _ptr(imp, ctypes.c_double), int(capacity))
    if rc != 0:
        raise ValueError("oracle importance: argument outside the method's domain")
    return imp


def max_threads(lib=None) -> int:
    return int((lib or load()).kvqo_max_threads())


def set_threads(n: int, lib=None) -> None:
    """Threads the oracle's attention loops use from now on."""
    (lib or load()).kvqo_set_threads(int(n))
