"""Batch-invariant verifier step of decode-verify-rollback inference on MI355X.

The HIP kernels live in libbiverify.so (C ABI: include/biverify.h); this
package is its ctypes binding (_lib) and the decoder-forward orchestration
that sequences those kernels (verifier).  There is no CPU or PyTorch
fallback: importing fails if the library has not been built.
"""
from ._lib import (  # noqa: F401
    ATTN_SEG_TOKENS,
    SWIGLU_BLOCK,
    BivError,
    abi_version,
    attn_adaptive_split,
    attn_decode_adaptive,
    attn_decode_bi,
    attn_decode_bi_static,
    ATTN_STATIC_SCRATCH_BYTES,
    attn_workspace_bytes,
    embed_rows,
    exported_symbols,
    gemm_bi,
    gemm_splitk,
    gumbel_topk,
    gumbel_verify,
    gumbel_workspace_bytes,
    kv_copy_pages,
    kv_overwrite,
    lm_head_gumbel_verify,
    pack_gate_up,
    rmsnorm_bi,
    rope_apply,
    rope_kv_overwrite,
    rope_table,
    splitk_auto_splits,
    splitk_workspace_bytes,
    swiglu,
    tree_select,
)
