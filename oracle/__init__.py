"""CPU float64 oracle for paged absorbed-MLA attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, links or calls anything in this package; only
the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the GPU path.

Every function states the passage of the source pages it follows.  Pages:

* "MLA Paged" (FlashInfer bench docs): the op definition, sections
  "prefill" and "decode" (axes, inputs, outputs, constraints).
* "flashinfer.attention.prims_ts.batch_mla_decode_with_paged_kv_cache"
  (FlashInfer API docs): host-side planning, ``mask_type``, ``seq_lens``.
* "mla_decoding_single_batch" (Modular MAX Mojo docs): V is the first
  ``depth_v`` dims of K; split-K stats ``exp_sum`` / ``qk_max``; the
  float8_e4m3fn query type.
* FlashMLA digest (context7 llms.txt): "Sparse MLA Prefill Kernel"
  (the written softmax-attention formula with lse), "FP8 KV Cache
  Quantization and Dequantization" / "... Utilities" (656-byte token record,
  block/offset slot mapping), "flash_mla_with_kvcache (Sparse Attention
  with FP8 KV Cache)" and "Sparse Attention Decoding with KV Cache" (token
  lists per query, the attention sink).

Pinning: every function here is checked by ``tests/test_oracle_*.py`` against
brute force, ``torch`` library routines in float64, closed forms and
invariants.  No function is "parity unpinned".
"""

from .mla_oracle import (  # noqa: F401
    HEAD_DIM_CKV,
    HEAD_DIM_KPE,
    FP8_RECORD_BYTES,
    bf16_bits_to_f64,
    as_f64,
    e4m3_decode,
    e4m3_encode,
    e4m3_all_finite_values,
    fp8_record_decode,
    fp8_record_encode,
    gather_request,
    gather_request_fp8,
    attend,
    attend_bruteforce,
    merge_partials,
    mla_decode_ref,
    mla_prefill_ref,
    mla_decode_fp8_ref,
    mla_decode_fp8_q8_ref,
    sparse_valid_indices,
    sparse_attend,
    mla_sparse_decode_fp8_ref,
    mla_sparse_prefill_ref,
    M1_NOPE,
    M1_RECORD_BYTES,
    f32_to_bf16_rne,
    model1_record_decode,
    model1_dequantize_bf16,
    model1_record_encode,
    mla_decode_model1_ref,
    mla_sparse_decode_model1_ref,
)
