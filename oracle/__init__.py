"""CPU oracle for quantized-KV append and decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP
library under ``decode_attention_quantized_append_amd``; neither imports the
other.

``oracle.core`` wraps the plain C codec and the exact double-precision
attention (``kvq_oracle.c``); ``oracle.cache_model`` is the cache model
(flat rows, the base-offset ring, truncate) written from the memra-engine
"Struct KvLayer" page (fields len_d, base_d, ring) and the "Struct Cache"
page (method rollback).
"""
from .core import (  # noqa: F401
    build_oracle, load, f32_to_f16, f16_to_f32, q8_0_encode, q8_0_decode,
    q5_1_encode, q5_1_decode, quantize_k, quantize_v, quantize_f8_rows, attention, max_threads,
    set_threads,
    widen_bf16,
)
from .cache_model import OracleCache, RangeError  # noqa: F401
