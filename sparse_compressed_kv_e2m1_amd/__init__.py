"""MI355X (gfx950) compressed sparse attention hot path: fp4 e2m1 round trips,
indexer scores + top-k, and sparse MQA attention with a per-head sink.

The computation lives in libsckv.so (hand-written HIP, C ABI in
include/sckv.h); this package is its ctypes binding (`_binding`, the same
call names) plus the per-step orchestration (`step.PathState`).  Importing
fails when libsckv.so has not been built.
"""
from ._binding import (  # noqa: F401
    SCKV_EHIP,
    SCKV_EINVAL,
    SCKV_EUNSUPPORTED,
    SCKV_EWORKSPACE,
    SCKV_FP4_E4M3_B16,
    SCKV_FP4_E8M0_B32,
    SCKV_OK,
    SCKV_OP_INDEX_SCORES_TOPK,
    SCKV_OP_INDEX_SCORES_TOPK_FP4,
    SCKV_OP_SPARSE_ATTN_SINK,
    LIB_PATH,
    SckvError,
    lib,
    sckv_abi_version,
    sckv_decode_prepare,
    sckv_decode_step,
    sckv_decode_step_workspace_bytes,
    sckv_index_scores_topk,
    sckv_index_scores_topk_fp4,
    sckv_last_error,
    sckv_prefill_prepare,
    sckv_quant,
    sckv_quant_pack,
    sckv_quant_rows,
    sckv_ring_write,
    sckv_rope_quant_pack,
    sckv_rope_quant_rows,
    sckv_rows_a_len,
    sckv_sparse_attn_sink,
    sckv_sparse_attn_sink_fp4,
    sckv_sparse_attn_sink_noalloc,
    sckv_sparse_attn_sink_noalloc_max_bytes,
    sckv_visible_idx,
    sckv_window_idx,
    sckv_workspace_bytes,
    sckv_yarn_freqs_cis,
    workspace,
)
