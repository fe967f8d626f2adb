"""kvq: append to, and decode attention over, a per-layer quantized KV cache
(K q8_0, V q5_1) on AMD Instinct MI355X (gfx950).

The product is the C-ABI library ``libkvq.so`` (header ``include/kvq.h``) built
from hand-written HIP kernels; ``kvq`` is its thin Python binding (argument
marshalling only) and ``KvqLayerCache`` a convenience owner of the device
buffers.  ``workloads`` holds seeded synthetic input generators.
"""
from .kvq import (  # noqa: F401
    EXPORTS, KVQ_BF16, KVQ_F32, KvqError, KvqLayerCache, kvq_append, kvq_create, kvq_decode,
    kvq_decode_workspace_bytes, kvq_destroy, kvq_host_lengths, kvq_info, kvq_last_error,
    kvq_required_bytes, kvq_set_split_rows, kvq_truncate, load, make_config,
)
