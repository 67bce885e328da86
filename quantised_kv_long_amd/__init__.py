"""Block-quantised KV-cache decode attention for AMD Instinct MI355X (gfx950).

The computation lives in ``libkvq.so`` (hand-written HIP kernels behind the C
ABI of include/kvq.h).  This package only binds it (``_lib``), allocates device
memory for it with torch (``cache``) and draws seeded synthetic inputs
(``synth``).
"""
from ._lib import (F16, OUT_F32, Q4_0, Q8_0, SPLIT_GRANULE, TYPES, KVQError, KVQLibraryMissing,
                   kvq_combine, kvq_data_row_bytes, kvq_decode_attn, kvq_decode_attn_variant,
                   kvq_plane_desc, kvq_quantize_append, kvq_scale_row_bytes, kvq_status_string,
                   load)

__all__ = ["F16", "Q8_0", "Q4_0", "OUT_F32", "SPLIT_GRANULE", "TYPES", "KVQError",
           "KVQLibraryMissing", "kvq_plane_desc", "kvq_data_row_bytes", "kvq_scale_row_bytes",
           "kvq_status_string", "kvq_quantize_append", "kvq_decode_attn",
           "kvq_decode_attn_variant", "kvq_combine", "load"]
