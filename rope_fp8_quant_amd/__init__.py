"""rope_fp8_quant_amd — the DSA-indexer Q/K preparation on MI355X (gfx950).

The computation lives in libdsaidx.so (hand-written HIP kernels behind a C ABI,
declared in include/dsaidx.h).  This package is its thin binding plus the
seeded synthetic workloads used to test and benchmark it.
"""
from .binding import (  # noqa: F401
    DSAIDX_ERR_HIP,
    DSAIDX_ERR_INVALID_ARGUMENT,
    DSAIDX_ERR_UNSUPPORTED,
    DSAIDX_K_BF16_INTERMEDIATE,
    DSAIDX_K_BF16_ROUND_ONCE,
    DSAIDX_K_PAGED_CACHE,
    DSAIDX_OK,
    DSAIDX_ROPE_INTERLEAVED,
    DSAIDX_ROPE_NEOX,
    DsaidxError,
    DsaidxKArgs,
    DsaidxLogitsArgs,
    DsaidxQArgs,
    DsaidxRope,
    dsaidx_abi_version,
    dsaidx_device_supported,
    dsaidx_fp8_encode_selftest,
    dsaidx_k_norm_rope_quant_store,
    dsaidx_k_only_prepare_store,
    dsaidx_mqa_logits,
    dsaidx_q_rope_quant_fold,
    dsaidx_qk_fused,
    dsaidx_status_string,
    dsaidx_topk_per_row,
    dsaidx_topk_per_row_noalloc,
    dsaidx_topk_workspace_bytes,
    k_args,
    lib,
    logits_args,
    q_args,
    rope_args,
)
