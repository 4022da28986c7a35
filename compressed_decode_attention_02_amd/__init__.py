"""TurboQuant KV-cache compression and packed-cache decode attention for MI355X (gfx950).

The compute path is the HIP library ``libtq.so`` (C ABI in ``include/tq.h``); this package
holds its sources (``csrc/``), the build script and the ctypes binding.
"""
from .binding import (  # noqa: F401
    EXPORTS, LIB_PATH, TQ_BF16, TQ_ERR_HIP, TQ_ERR_INVALID_ARG, TQ_ERR_RING_FULL, TQ_ERR_SCRATCH_LIMIT,
    TQ_ERR_UNSUPPORTED, TQ_ERR_WORKSPACE, TQ_F16, TQ_F32, TQ_NOALLOC_SCRATCH_BYTES, TQ_OK, PackedStore, PagedStore,
    PreparedDecodeStep, Ring, Tables, TqError, lib, make_config, new_workspace, tq_append_ring, tq_build_codebook,
    tq_build_rotation, tq_build_tables, tq_config, tq_decode_attention, tq_decode_attention_noalloc,
    tq_decode_attention_ragged, tq_decode_scores, tq_decode_step, tq_decode_workspace_bytes, tq_flush, tq_packed,
    tq_packed_bytes_per_token, tq_quantize_kv, tq_ring, tq_rotate, tq_tables, tq_tables_bytes,
    tq_prefill_attention, tq_prefill_workspace_bytes, new_prefill_workspace, key_record_words,
    KiviStore, tq_kivi_store, tq_kivi_bytes_per_token, tq_kivi_quantize, tq_kivi_decode_workspace_bytes,
    tq_kivi_decode_attention, new_kivi_workspace,
)
