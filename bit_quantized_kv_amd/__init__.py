"""4-bit paged KV cache (TQ4/4, MX-FP4) and decode attention over the
compressed cache, as HIP kernels for AMD MI355X (gfx950).

The C ABI is ``include/tq.h`` (``libtq.so``); ``binding`` exposes it under the
same names, and ``Cache`` is a small convenience wrapper that keeps the pool
and the workspace in torch tensors.
"""
from .binding import (  # noqa: F401
    TQ_FORMAT_MXFP4, TQ_FORMAT_TQ4, TQ_FORMAT_TQ4V2, TQ_OUT_BF16, TQ_OUT_F32, TqError, tq_cache_info, tq_create_cache,
    tq_decode_attention, tq_decode_workspace_bytes, tq_default_key_table, tq_free, tq_pool_bytes,
    tq_quantize_append, tq_record_bytes, tq_calibrate_workspace_bytes, tq_calibrate_key_tables, tq_select_layers,
    tq_multitoken_workspace_bytes, tq_multitoken_attention, tq_cascade_workspace_bytes, tq_cascade_decode_attention,
)
from .cache import Cache, CascadeGroups, calibrate_key_tables  # noqa: F401
