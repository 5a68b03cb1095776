"""Paged absorbed-MLA attention for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libmla.so`` (declared in
``include/mla.h``).  It only marshals arguments: allocation of outputs and
workspace goes through torch, every step of the computation runs in the
library's HIP kernels.  If the library is missing or cannot be loaded, every
call raises; there is no fallback.

Names follow the C ABI: :func:`mla_plan_create`, :func:`mla_decode`,
:func:`mla_prefill`, the capacity-plan :func:`mla_decode_live` /
:func:`mla_prefill_live`, :func:`mla_decode_fp8`, :func:`mla_decode_fp8_q8` (e4m3
query), :func:`mla_decode_noalloc` (no device allocation), the concatenated-layout
:func:`mla_decode_packed` / :func:`mla_prefill_packed`,
:func:`mla_block_table_to_indices`, and the token-sparse
:func:`mla_sparse_plan_create` / :func:`mla_sparse_decode_fp8` /
:func:`mla_sparse_prefill`.
"""

from ._binding import (  # noqa: F401
    MLAError,
    Plan,
    lib_path,
    load_library,
    mla_block_table_to_indices,
    mla_decode,
    mla_decode_fp8,
    mla_decode_fp8_q8,
    mla_decode_live,
    mla_decode_model1,
    mla_decode_noalloc,
    mla_decode_packed,
    mla_model1_expand_q,
    mla_model1_expand_records,
    mla_plan_create,
    mla_prefill,
    mla_prefill_live,
    mla_prefill_packed,
    mla_record_attention_events,
    mla_sparse_decode_fp8,
    mla_sparse_decode_model1,
    mla_sparse_plan_create,
    mla_sparse_prefill,
    MLA_KIND_DECODE,
    MLA_KIND_PREFILL,
    MLA_KIND_SPARSE_DECODE,
    MLA_KV_BF16,
    MLA_KV_FP8_E4M3_T128,
    MLA_KV_FP8_MODEL1,
    MLA_LSE_ROWS,
    MLA_LSE_HEADS_FIRST,
    MLA_ERR_INVALID_ARGUMENT,
    MLA_TILE_AUTO,
    MLA_TILE_WIDE,
    MLA_TILE_NARROW,
    MLA_TILE_QUAD,
    MODEL1_NOPE,
    MODEL1_RECORD,
    NOALLOC_SCRATCH_BYTES,
)
