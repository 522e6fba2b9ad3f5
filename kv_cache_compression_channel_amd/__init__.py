"""libkvq: KV-cache compression hot path for AMD Instinct MI355X (gfx950).

Per-channel INT8, KIVI-style INT4 group quantization with a bf16 residual window,
dequantization, error statistics, INT4 GQA decode attention, H2O / SnapKV token
selection and compaction -- hand-written HIP kernels behind a C ABI (include/kvq.h),
with this package as a thin ctypes binding.
"""
from .kvq import (  # noqa: F401
    EXPORTED,
    Int4Cache,
    KVQError,
    compact,
    compression_ratio,
    decode_attn_int4,
    dequant_int4,
    dequant_pc,
    err_stats,
    group_quant_int4,
    h2o_select,
    int4_bytes,
    int4_cache_sizes,
    keep_count,
    kv_bytes,
    lib,
    quant_asym,
    quant_sym,
    snapkv_select,
    stats_finalize,
    token_ratio,
    total_gain,
)
