"""Hybrid-attention decode step for MI355X (gfx950).

One decode step of a hybrid model (full-attention layers interleaved with
Gated DeltaNet layers) behind a small C ABI (``include/had.h``,
``libhad.so``): the paged KV-cache / state-slot manager, the fused
QK-RMSNorm + partial-RoPE + gate-split prologue, split-K GQA decode
attention and the slot-addressed gated delta rule update.  This package is
the thin Python binding over that library; torch supplies device memory and
streams.
"""

from ._lib import (  # noqa: F401
    HadError,
    PageTable,
    RadixCache,
    SlotPool,
    abi_version,
    attn_check_prefix,
    attn_desc,
    decode_attn,
    decode_attn_cascade,
    decode_attn_cascade_combine,
    decode_attn_cascade_partial,
    decode_attn_cascade_plan,
    decode_attn_cascade_workspace_bytes,
    decode_attn_combine,
    decode_attn_layer,
    decode_attn_layer_static,
    decode_attn_partial,
    decode_attn_plan,
    decode_attn_workspace_bytes,
    exported_symbols,
    gdn_check_slots,
    gdn_prefill,
    gdn_prefill_desc,
    gdn_prefill_workspace_bytes,
    gdn_state_update,
    kv_append,
    kv_check_copy_pages,
    kv_copy_pages,
    lib,
    qk_norm_rope_gate,
    spec_rollback,
    DERR_PAGE,
    DERR_SLOT,
    DERR_SEQLEN,
    DERR_COPY,
)
