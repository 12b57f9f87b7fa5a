"""Batch-invariant causal GQA attention over a paged KV cache for MI355X (gfx950).

The compute path is the HIP library ``libbiattn.so`` (C ABI in ``include/bi_attn.h``);
this package is its thin binding (``_lib``) plus the build step (``build``).
"""

from ._lib import (  # noqa: F401
    AttnConfig,
    BiAttnError,
    BI_BF16,
    BI_F32,
    BI_SPLIT_BY_BATCH,
    BI_SPLIT_BY_BATCH_FILL,
    BI_SPLIT_FIXED,
    EXPORTED,
    LIB_PATH,
    bi_attn_decode,
    bi_attn_decode_noalloc,
    NOALLOC_SCRATCH_BYTES,
    bi_gemm,
    bi_attn_decode_append,
    bi_attn_decode_append_partials,
    bi_attn_decode_combine,
    bi_attn_decode_partials,
    bi_attn_prefill,
    bi_attn_varlen,
    bi_attn_workspace_bytes,
    bi_kv_page_update,
    bi_rmsnorm,
    bi_status_string,
    load,
)
