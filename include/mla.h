/*
 * mla.h — C ABI of the paged absorbed-MLA attention library (libmla.so),
 * built for AMD Instinct MI355X (gfx950) with hand-written HIP kernels.
 *
 * The operation ("MLA Paged", FlashInfer bench docs, sections "decode" and
 * "prefill"): for each query row r and head h,
 *     s_j  = sm_scale * (q_nope[r,h,:] . ckv_j + q_pe[r,h,:] . kpe_j)
 *     lse  = ln sum_j exp(s_j)                     (natural log, fp32)
 *     out  = sum_j exp(s_j - lse) * ckv_j          (V = first 512 latent dims,
 *                                                   "mla_decoding_single_batch")
 * over the keys j the row may see, gathered through the page table
 * kv_indptr / kv_indices from [num_pages, page_size, dim] caches.  The
 * log-sum-exp / exp(P - lse) form is the one written in FlashMLA's "Sparse
 * MLA Prefill Kernel" passage (there in base 2; here natural log).
 *
 * Conventions for every call below
 *   - Pointers named *_host are host memory; every other array pointer is
 *     device memory on the current HIP device.  All tensors are dense,
 *     row-major and contiguous with the shapes given.
 *   - bf16 means IEEE-754 binary32 truncated to its upper 16 bits
 *     (bfloat16), little-endian; int32 arrays are little-endian.
 *   - The caller owns every device buffer (inputs, out, lse, workspace) and
 *     the stream.  The library owns only the host-side plan object.
 *   - No call throws.  Every call returns an mla_status; on error nothing is
 *     launched and no output is written.
 *   - Run calls (mla_decode, mla_prefill, mla_decode_fp8 and the others)
 *     allocate nothing, never synchronise and never copy to or from the host:
 *     they only enqueue kernels on `stream`, so they can be captured into a
 *     HIP graph.  The one exception is a plan made with validate = 1, whose
 *     run calls read the device index arrays' check result back (one
 *     synchronisation of `stream`) before launching.  Calls that overlap in
 *     time must use different workspaces.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = -1, /* null pointer, bad size, inconsistent host arrays */
  MLA_ERR_UNSUPPORTED = -2,      /* a shape or mode this library does not implement   */
  MLA_ERR_WORKSPACE = -3,        /* workspace missing, misaligned or too small        */
  MLA_ERR_PLAN_MISMATCH = -4,    /* run call does not match the plan's kind / format  */
  MLA_ERR_DEVICE = -5            /* a HIP runtime call or kernel launch failed        */
} mla_status;

typedef enum mla_dtype { MLA_DTYPE_BF16 = 0, MLA_DTYPE_FP32 = 1 } mla_dtype;

/* Latent-cache formats.
 *   MLA_KV_BF16: two caches, ckv [num_pages, page_size, 512] bf16 and
 *     kpe [num_pages, page_size, 64] bf16 ("MLA Paged", Inputs).
 *   MLA_KV_FP8_E4M3_T128: one cache [num_pages, page_size, 656] uint8, one
 *     656-byte record per token (FlashMLA digest, "FP8 KV Cache Quantization
 *     and Dequantization", V32_FP8Sparse): bytes 0..511 = 512 OCP e4m3
 *     codes of the latent dims, bytes 512..527 = four little-endian fp32
 *     scales (scale t applies to dims 128t..128t+127), bytes 528..655 = the
 *     64 rope dims as bf16.  Key value = code * scale; rope as stored.
 *   MLA_KV_FP8_MODEL1: one cache [num_pages, page_size, 604] uint8, one
 *     604-byte MODEL1 record per token (same page, MODEL1_FP8Sparse: d = 512
 *     for q.k, 448 NoPE dims in 7 tiles of 64, 64 RoPE dims; the page gives
 *     sizes only, the byte order read here is the printed one, packed):
 *     bytes 0..447 = e4m3 codes (tile t = dims 64t..64t+63), bytes 448..475
 *     = seven little-endian fp32 scales, bytes 476..603 = the 64 RoPE dims
 *     as bf16.  Key value = code * scale, exactly as for the 656-byte
 *     records; V = the 448 NoPE dims.  Decode only (mla_decode_model1,
 *     mla_sparse_decode_model1); no quad tile.                            */
typedef enum mla_kv_format {
  MLA_KV_BF16 = 0,
  MLA_KV_FP8_E4M3_T128 = 1,
  MLA_KV_FP8_MODEL1 = 2
} mla_kv_format;

/* MLA_KIND_SPARSE_DECODE: plans made by mla_sparse_plan_create only. */
typedef enum mla_kind { MLA_KIND_DECODE = 0, MLA_KIND_PREFILL = 1, MLA_KIND_SPARSE_DECODE = 2 } mla_kind;

/* Tile modes of the attention kernel (0 lets the planner choose: WIDE when
 * some request holds at least 64 query rows (heads x query tokens), NARROW
 * otherwise).
 *   MLA_TILE_WIDE:   a workgroup holds up to 128 query rows, 32 per wave, and
 *                    all four waves share each key tile.
 *   MLA_TILE_NARROW: a workgroup holds up to 16 query rows and its four waves
 *                    split every key tile between them.
 *   MLA_TILE_QUAD:   a workgroup holds 32 rows; its waves split each key tile
 *                    for Q.K^T and the 512 output columns for P.V; up to four
 *                    sibling workgroups on one XCD hold the other 32-row
 *                    slices of the same rows and walk the same keys (bf16 caches only).  */
typedef enum mla_tile_mode {
  MLA_TILE_AUTO = 0,
  MLA_TILE_WIDE = 1,
  MLA_TILE_NARROW = 2,
  MLA_TILE_QUAD = 3
} mla_tile_mode;

/* Layouts of the lse output.
 *   MLA_LSE_ROWS:        [rows, H] fp32, row = query token (the layout of
 *                        "MLA Paged", decode and prefill outputs).
 *   MLA_LSE_HEADS_FIRST: [batch, H, s_q] fp32, every request holding the
 *                        same number s_q of query tokens (the lse of FlashMLA's
 *                        "flash_mla_with_kvcache (Dense Attention)", batch x
 *                        num_heads_q x seq_len_q); decode has s_q = 1, where
 *                        both layouts coincide.                            */
typedef enum mla_lse_layout { MLA_LSE_ROWS = 0, MLA_LSE_HEADS_FIRST = 1 } mla_lse_layout;

typedef struct mla_plan_desc {
  int32_t kind;          /* mla_kind                                                */
  int32_t batch;         /* number of requests, >= 0                                */
  int32_t num_qo_heads;  /* query heads H, >= 1 (the latent cache has one KV head) */
  int32_t head_dim_ckv;  /* must be 512                                             */
  int32_t head_dim_kpe;  /* must be 64                                              */
  int32_t page_size;     /* tokens per page, a power of two in [1, 4096]            */
  int32_t num_pages;     /* pages in the cache pool, >= 1                           */
  int32_t kv_format;     /* mla_kv_format                                           */
  int32_t causal;        /* prefill only: 1 = causal, bottom-right aligned; 0 = none */
  int32_t num_cus;       /* compute units to balance for; 0 = ask the current device */
  int32_t max_splits;    /* upper bound on key chunks per request; 0 = automatic    */
  int32_t force_splits;  /* > 0: cut every request into this many chunks (testing)  */
  int32_t tile_mode;     /* mla_tile_mode                                           */
  int32_t validate;      /* 1: every run call first checks the device index arrays
                            against the plan on the device, synchronises the stream
                            and returns MLA_ERR_INVALID_ARGUMENT before any attention
                            launch if one is wrong (not capture-safe); 0: no check */
  int32_t lse_layout;    /* mla_lse_layout                                          */
  int32_t max_kv_len;    /* > 0: a capacity plan for any live key counts in
                            [0, max_kv_len] (runs take them on the device)         */
  int32_t max_seq_len_q; /* capacity plans, prefill: query tokens per request,
                            >= every live q_len (0: the largest qo_indptr delta)  */
} mla_plan_desc;

typedef struct mla_plan mla_plan; /* opaque, immutable after creation */

/* Host-side plan: the split-KV schedule for one set of request lengths.
 * Follows the planning step the pages describe: FlashMLA's
 * "get_mla_metadata" (computed once before the decode loop, reusable across
 * layers while cache_seqlens are unchanged) and FlashInfer's
 * "batch_mla_decode_with_paged_kv_cache" (the host reads seq_lens and
 * qo_indptr to derive plan bounds; run outside graph capture).
 *
 *   kv_len_host    [batch]   int32: keys of each request (the pages'
 *                  seq_lens / cache_seqlens).  NULL means every page of the
 *                  request is full: kv_len = pages * page_size.
 *   kv_indptr_host [batch+1] int32: the same CSR offsets that will be passed
 *                  to the run call; kv_indptr[b+1]-kv_indptr[b] must equal
 *                  ceil(kv_len[b] / page_size) and kv_indptr[0] must be 0.
 *   qo_indptr_host [batch+1] int32, prefill only (else NULL): query row
 *                  offsets, qo_indptr[0] = 0, non-decreasing; with causal=1
 *                  each request needs q_len <= kv_len.
 * The plan is valid for any call with the same lengths and descriptor.
 *
 * Capacity plans (desc.max_kv_len > 0; "batch_mla_decode_with_paged_kv_cache",
 * Parameters: max_kv_len, the static K/V length bound, and max_seq_len_q, the
 * per-request packed-query capacity, which may exceed the live lengths): the
 * schedule is made as if every request had max_kv_len keys and, for prefill,
 * max_seq_len_q query tokens (0: the largest delta of qo_indptr_host), with no
 * causal trimming, so one plan serves every step whose live lengths stay
 * within those bounds.  kv_len_host and kv_indptr_host are then ignored (may
 * be NULL), and so is qo_indptr_host when max_seq_len_q > 0.  The live
 * lengths go to mla_decode_live / mla_prefill_live on the device; work past
 * them is skipped in the kernels.  Other run calls refuse capacity plans
 * (MLA_ERR_PLAN_MISMATCH), and capacity plans are bf16 only.
 *
 * lse_layout MLA_LSE_HEADS_FIRST needs every request to have the same number
 * of query tokens (capacity prefill: max_seq_len_q of them, live counts may
 * be smaller); rows past a request's live tokens are left unwritten.
 *
 * Errors: MLA_ERR_INVALID_ARGUMENT (null pointers, inconsistent arrays,
 * max_kv_len or max_seq_len_q < 0, unequal query counts with
 * MLA_LSE_HEADS_FIRST, validate not 0 or 1), MLA_ERR_UNSUPPORTED (head dims
 * other than 512/64, page_size not a power of two in range, fp8 prefill, an
 * fp8 capacity plan), MLA_ERR_DEVICE (num_cus = 0 and the device query
 * failed).  Makes no device allocation and launches nothing.             */
mla_status mla_plan_create(mla_plan** plan, const mla_plan_desc* desc,
                           const int32_t* kv_len_host, const int32_t* kv_indptr_host,
                           const int32_t* qo_indptr_host);

void mla_plan_destroy(mla_plan* plan);

/* Bytes of device workspace the run calls need with this plan (work list,
 * split partial outputs and their lse), and the number of work items and of
 * split groups (diagnostics).                                             */
size_t mla_plan_workspace_bytes(const mla_plan* plan);
int32_t mla_plan_num_work_items(const mla_plan* plan);
int32_t mla_plan_num_split_groups(const mla_plan* plan);

/* Copy the plan's work list [num_work_items][8] int32 to host memory
 * `items_host` (test and diagnostic use): per item
 *   {request, first_row, num_rows, key_begin, key_end, kv_len, q_len, slot}
 * where rows count (query token, head) pairs of the request as
 * token * H + head and slot is -1 for an item that writes the final output
 * or the index of its partial-result slot.                               */
mla_status mla_plan_get_work_items(const mla_plan* plan, int32_t* items_host, size_t capacity);

/* Work lists of the attention kernel: list w holds work items
 * wg_ptr[w] .. wg_ptr[w+1]-1, processed in order by one workgroup (by each
 * of mla_plan_group_size sibling workgroups in the quad tile mode, sibling r
 * taking rows 32r..32r+31 of every item).  mla_plan_get_workgroup_ptr copies
 * the [num_workgroups + 1] int32 offsets to host memory (diagnostics).    */
int32_t mla_plan_num_workgroups(const mla_plan* plan);
int32_t mla_plan_group_size(const mla_plan* plan);
mla_status mla_plan_get_workgroup_ptr(const mla_plan* plan, int32_t* wg_ptr_host, size_t capacity);

/* One asynchronous host-to-device copy of the plan's work list into the
 * head of `workspace` (device memory of at least mla_plan_workspace_bytes,
 * 256-byte aligned) on `stream`.  Must be called (outside graph capture)
 * before the first run call that uses this workspace with this plan.      */
mla_status mla_plan_upload(const mla_plan* plan, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Decode ("MLA Paged", section "decode"): one query row per request.
 *   q_nope [batch, H, 512] bf16; q_pe [batch, H, 64] bf16
 *   ckv_cache [num_pages, page_size, 512] bf16; kpe_cache [num_pages, page_size, 64] bf16
 *   kv_indptr [batch+1] int32 (device copy of the plan's), kv_indices
 *   [kv_indptr[batch]] int32 page ids in [0, num_pages)
 *   sm_scale: scale applied to q.k ("softmax scale", finite)
 *   out [batch, H, 512] of out_dtype (bf16 or fp32); lse [batch, H] fp32,
 *   natural log; a request with kv_len 0 gets out = 0 and lse = -inf.
 * Slots past kv_len in a request's last page and pages no request lists
 * are never read into the result (they may hold any bits, NaN included).
 * Errors: MLA_ERR_INVALID_ARGUMENT (null pointer, non-finite sm_scale, bad
 * out_dtype; with validate = 1 also kv_indptr unequal to the plan's or a page
 * id outside [0, num_pages)), MLA_ERR_PLAN_MISMATCH (plan is not a bf16
 * decode plan, or is a capacity plan), MLA_ERR_WORKSPACE, MLA_ERR_DEVICE
 * (launch failed).                                                       */
mla_status mla_decode(const mla_plan* plan, const void* q_nope, const void* q_pe,
                      const void* ckv_cache, const void* kpe_cache, const int32_t* kv_indptr,
                      const int32_t* kv_indices, float sm_scale, void* out, int32_t out_dtype,
                      float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Prefill ("MLA Paged", section "prefill"): packed query rows, request b
 * owning rows qo_indptr[b] .. qo_indptr[b+1]-1, total_q = qo_indptr[batch].
 *   q_nope [total_q, H, 512] bf16; q_pe [total_q, H, 64] bf16
 *   qo_indptr [batch+1] int32 (device copy of the plan's)
 *   out [total_q, H, 512]; lse [total_q, H] fp32.
 * With causal=1 (the default mask_type of "batch_mla_decode_with_paged_kv_cache"),
 * query i of a request with n queries and L keys sees keys 0..L-n+i.
 * Everything else as for mla_decode; the plan must be a bf16 prefill plan. */
mla_status mla_prefill(const mla_plan* plan, const void* q_nope, const void* q_pe,
                       const void* ckv_cache, const void* kpe_cache, const int32_t* qo_indptr,
                       const int32_t* kv_indptr, const int32_t* kv_indices, float sm_scale,
                       void* out, int32_t out_dtype, float* lse, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* Run calls of capacity plans (desc.max_kv_len > 0): as mla_decode /
 * mla_prefill, with the live key counts on the device.
 *   kv_len [batch] int32 device: keys of each request this step, each in
 *     [0, max_kv_len] (the pages' seq_lens / cache_seqlens);
 *   kv_indptr [batch+1] int32 device: page offsets of this step, with
 *     kv_indptr[b+1] - kv_indptr[b] >= ceil(kv_len[b] / page_size);
 *   qo_indptr [batch+1] int32 device (prefill): query offsets of this step,
 *     every delta <= max_seq_len_q, with delta <= kv_len[b] when causal.
 * Rows of a request past its live query tokens are not written (their lse
 * entries included); a request with kv_len 0 gets out 0 and lse -inf.
 * Out-of-bound live lengths are caught by validate = 1; without it a live
 * count above the plan's bound is treated as the bound.  Errors as for
 * mla_decode, plus MLA_ERR_PLAN_MISMATCH for a plan that is not a capacity
 * plan of the call's kind.                                               */
mla_status mla_decode_live(const mla_plan* plan, const void* q_nope, const void* q_pe, const void* ckv_cache,
                           const void* kpe_cache, const int32_t* kv_len, const int32_t* kv_indptr,
                           const int32_t* kv_indices, float sm_scale, void* out, int32_t out_dtype, float* lse,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);
mla_status mla_prefill_live(const mla_plan* plan, const void* q_nope, const void* q_pe, const void* ckv_cache,
                            const void* kpe_cache, const int32_t* qo_indptr, const int32_t* kv_len,
                            const int32_t* kv_indptr, const int32_t* kv_indices, float sm_scale, void* out,
                            int32_t out_dtype, float* lse, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Decode over the fp8 record cache (MLA_KV_FP8_E4M3_T128 above):
 *   kv_cache [num_pages, page_size, 656] uint8; q_nope / q_pe bf16 as in
 *   mla_decode.  Keys are dequantised in the kernel ("FP8 KV Cache
 *   Quantization and Dequantization" of the FlashMLA digest): each code is
 *   converted exactly, each 128-dim tile's partial dot product is scaled by
 *   the key's fp32 tile scale, and P is scaled per key before P.V; everything
 *   else as for mla_decode.  Plan: fp8 decode plan.                       */
mla_status mla_decode_fp8(const mla_plan* plan, const void* q_nope, const void* q_pe,
                          const void* kv_cache, const int32_t* kv_indptr,
                          const int32_t* kv_indices, float sm_scale, void* out,
                          int32_t out_dtype, float* lse, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Decode over the fp8 record cache with an fp8 query ("mla_decoding_single_batch":
 * q_type float8_e4m3fn, bfloat16 output):
 *   q [batch, H, 576] uint8: OCP e4m3 codes of the query, latent dims then
 *     rope dims, used as they are (no scale; the caller quantises).
 * The product over the 512 latent dims runs on the fp8 x fp8 matrix cores
 * (per-tile key scales applied in fp32 as in mla_decode_fp8); the rope dims
 * and P.V are as in mla_decode_fp8.  The hardware sums each 64-deep block of
 * code products with a limited alignment window (measured: error below
 * 2e-5 of the sum of the products' magnitudes), so the logits are exact to
 * that bound rather than to fp32 rounding.  Plan: an fp8 decode plan in
 * the WIDE tile mode (another mode is MLA_ERR_UNSUPPORTED).  Everything
 * else, errors included, as for mla_decode_fp8.                          */
mla_status mla_decode_fp8_q8(const mla_plan* plan, const void* q, const void* kv_cache,
                             const int32_t* kv_indptr, const int32_t* kv_indices, float sm_scale, void* out,
                             int32_t out_dtype, float* lse, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* The concatenated layout ("MLA Paged" ckv/kpe as one tensor; FlashMLA's
 * "flash_mla_with_kvcache" q and k_cache with head_dim 576): one 576-wide
 * bf16 row per query (token, head) and per cached token, latent dims 0..511
 * then rope dims 512..575.
 *   q [rows, H, 576] bf16 (rows = batch for decode, total_q for prefill)
 *   kv_cache [num_pages, page_size, 576] bf16
 *   out_scale: factor applied to every output row (the output scaling of
 *   "batch_mla_decode_with_paged_kv_cache", bmm2_scale); lse is unchanged.
 * Everything else, errors included (a non-finite out_scale is
 * MLA_ERR_INVALID_ARGUMENT), as for mla_decode / mla_prefill; the same
 * bf16 plans serve both layouts, and with out_scale = 1 the results are
 * bit-identical to the split layout's.                                   */
mla_status mla_decode_packed(const mla_plan* plan, const void* q, const void* kv_cache,
                             const int32_t* kv_indptr, const int32_t* kv_indices, float sm_scale,
                             float out_scale, void* out, int32_t out_dtype, float* lse, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);
mla_status mla_prefill_packed(const mla_plan* plan, const void* q, const void* kv_cache,
                              const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                              float sm_scale, float out_scale, void* out, int32_t out_dtype, float* lse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Dense block tables ("batch_mla_decode_with_paged_kv_cache" block_tables,
 * FlashMLA block_table) to the page lists of the run calls: enqueues on
 * `stream` kv_indices[kv_indptr[b] + j] = block_table[b * max_blocks + j]
 * for j < kv_indptr[b+1] - kv_indptr[b] (the pages the plan's lengths
 * need; later table entries are padding and are not read).
 *   block_table [batch, max_blocks] int32 device; kv_indptr [batch+1]
 *   int32 device, equal to the plan's; kv_indices [kv_indptr[batch]] int32
 *   device, written.
 * Errors: MLA_ERR_INVALID_ARGUMENT (null pointer, max_blocks < 0 or smaller
 * than a request's page count), MLA_ERR_DEVICE (launch failed).  Allocates
 * nothing; capture-safe.                                                 */
mla_status mla_block_table_to_indices(const mla_plan* plan, const int32_t* block_table, int32_t max_blocks,
                                      const int32_t* kv_indptr, int32_t* kv_indices, hipStream_t stream);

/* Decode over MODEL1 records (MLA_KV_FP8_MODEL1 above), dequantised in the
 * kernel as the 656-byte records are: codes converted exactly, each 64-dim
 * tile's partial dot product scaled by the key's fp32 tile scale, P scaled
 * per key by the output tile's scale before P.V.
 *   q [batch, H, 512] bf16: 448 NoPE dims, then 64 RoPE dims
 *   kv_cache [num_pages, page_size, 604] uint8
 *   out [batch, H, 512] of out_dtype: dims 0..447 the attention output
 *     (V = the 448 NoPE dims), dims 448..511 written as 0; lse [batch, H].
 * Plan: a decode plan with kv_format MLA_KV_FP8_MODEL1.  Everything else,
 * errors included, as for mla_decode_fp8.
 *
 * mla_sparse_decode_model1: token-sparse decode over MODEL1 records, as
 * mla_sparse_decode_fp8 with q [num_tokens, H, 512] (448 NoPE + 64 RoPE),
 * kv_cache [num_slots, 604] records and out [num_tokens, H, 512] (dims
 * 448..511 written as 0); plan: mla_sparse_plan_create with
 * MLA_KV_FP8_MODEL1.                                                      */
mla_status mla_decode_model1(const mla_plan* plan, const void* q, const void* kv_cache, const int32_t* kv_indptr,
                             const int32_t* kv_indices, float sm_scale, void* out, int32_t out_dtype, float* lse,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);
mla_status mla_sparse_decode_model1(const mla_plan* plan, const void* q, const void* kv_cache,
                                    const int32_t* indices, const int32_t* topk_length, const float* attn_sink,
                                    float sm_scale, void* out, int32_t out_dtype, float* lse, float* max_logits,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The page's BF16 dequantisation of MODEL1 records ("FP8 KV Cache
 * Quantization Utilities", dequantize_k_cache returns the BF16 cache), as a
 * layout utility: value = bf16(fp32(code) * scale), both steps round to
 * nearest even.  These rows are not what mla_decode_model1 attends over
 * (it uses the exact products); attention over them is attention over the
 * BF16-rounded keys.
 *
 * mla_model1_expand_records: records [num_tokens, 604] (u8, device, 4-byte
 * aligned) -> rows [num_tokens, 576] (bf16, device, 16-byte aligned) in the
 * concatenated layout of mla_decode_packed / mla_prefill_packed /
 * mla_sparse_prefill: dims 0..447 the dequantised NoPE values, 448..511
 * zero, 512..575 the RoPE values.  num_tokens counts every record of the
 * array (a paged pool is num_pages * page_size records, kept in order).
 * mla_model1_expand_q: query rows [num_rows, 512] (bf16: 448 NoPE + 64
 * RoPE, 16-byte aligned) -> [num_rows, 576] the same way.
 * With both expanded, attention through the 576-wide calls is the MODEL1
 * attention (q.k over 512 dims); the first 448 output dims are its output
 * (V = the 448 NoPE dims) and dims 448..511 come out 0.
 * Errors: MLA_ERR_INVALID_ARGUMENT (num_tokens / num_rows < 0, a null or
 * misaligned pointer with a non-zero count), MLA_ERR_DEVICE (launch
 * failed).  The caller owns every buffer; nothing is allocated; enqueued on
 * `stream` only (capture-safe).                                          */
mla_status mla_model1_expand_records(const uint8_t* records, int64_t num_tokens, void* rows, hipStream_t stream);
mla_status mla_model1_expand_q(const void* q, int64_t num_rows, void* q576, hipStream_t stream);

/* Token-sparse attention (DSA) over the 656-byte fp8 record cache
 * (mla_sparse_decode_fp8: FlashMLA digest, "flash_mla_with_kvcache (Sparse
 * Attention with FP8 KV Cache)" and "Sparse Attention Decoding with KV
 * Cache") or over bf16 576-wide KV rows (mla_sparse_prefill: "Sparse MLA
 * Prefill Kernel", flash_mla_sparse_fwd); the formula of "Sparse MLA
 * Prefill Kernel".  Every query token t has its own list of key slots;
 * for each head h:
 *   s_j = sm_scale * (q[t,h,:512] . nope_j + q[t,h,512:] . rope_j) over the
 *         valid entries j of indices[t, :], nope_j = code * tile scale;
 *   max_logits[t,h] = max_j s_j,  lse[t,h] = ln sum_j exp(s_j),
 *   out[t,h] = sum_j exp(s_j) nope_j / (sum_j exp(s_j) + exp(attn_sink[h]))
 *   (without attn_sink: the plain softmax average).  No valid entry: out 0,
 *   lse and max_logits -inf.
 *
 * mla_sparse_plan_create: the schedule for num_tokens query tokens of
 * num_heads heads, each with a list of topk entries into a pool of
 * num_slots key rows (fp8: num_blocks * block_size records), for kv_format
 * MLA_KV_FP8_E4M3_T128 (mla_sparse_decode_fp8) or MLA_KV_BF16
 * (mla_sparse_prefill).  Work is balanced as if every
 * entry were valid.  num_cus = 0 asks the current device; force_splits > 0
 * cuts every list into that many chunks (testing).  Errors:
 * MLA_ERR_INVALID_ARGUMENT (sizes < 1 where 1 is needed, force_splits < 0,
 * num_tokens * topk >= 2^31), MLA_ERR_UNSUPPORTED (another kv_format),
 * MLA_ERR_DEVICE (device query failed).  The workspace holds the compacted
 * lists; its size is mla_plan_workspace_bytes and it is uploaded with
 * mla_plan_upload like any plan's.
 *
 * mla_sparse_decode_fp8 arguments (device pointers unless noted):
 *   q          [num_tokens, H, 576] bf16, latent dims then rope dims (the
 *              pages' q [batch, s_q, H, 576] with batch and s_q flattened)
 *   kv_cache   [num_slots, 656] uint8 records (a [num_blocks, block_size,
 *              (1,) 656] cache viewed flat)
 *   indices    [num_tokens, topk] int32 flat slots block * block_size +
 *              offset; -1, a negative value or a slot >= num_slots is an
 *              invalid entry and is skipped; a slot listed twice counts twice
 *   topk_length [num_tokens] int32 or NULL: only the first
 *              min(topk_length[t], topk) entries of row t are used
 *   attn_sink  [H] fp32 or NULL: per-head sink logit (natural-log units)
 *   out        [num_tokens, H, 512] bf16 or fp32 (out_dtype); lse and
 *              max_logits [num_tokens, H] fp32 (max_logits may be NULL)
 * mla_sparse_prefill takes the same arguments with
 *   kv         [num_slots, 576] bf16 rows (latent dims then rope dims; the
 *              page's kv [s_kv, h_kv = 1, 576]), indices into its rows
 *   q          [num_tokens, H, 576] bf16 (the page's q [s_q, H, 576])
 * The lists are compacted into the workspace on `stream` first, so the
 * workspace may not be shared by calls that overlap.  Errors as for
 * mla_decode; a plan not made by mla_sparse_plan_create for the call's
 * cache format is MLA_ERR_PLAN_MISMATCH.  Allocates nothing and never
 * synchronises.                                                          */
mla_status mla_sparse_plan_create(mla_plan** plan, int32_t num_tokens, int32_t num_heads, int32_t num_slots,
                                  int32_t topk, int32_t kv_format, int32_t num_cus, int32_t force_splits);
mla_status mla_sparse_decode_fp8(const mla_plan* plan, const void* q, const void* kv_cache, const int32_t* indices,
                                 const int32_t* topk_length, const float* attn_sink, float sm_scale, void* out,
                                 int32_t out_dtype, float* lse, float* max_logits, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);
mla_status mla_sparse_prefill(const mla_plan* plan, const void* q, const void* kv, const int32_t* indices,
                              const int32_t* topk_length, const float* attn_sink, float sm_scale, void* out,
                              int32_t out_dtype, float* lse, float* max_logits, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* mla_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and kernels as mla_decode, with the workspace taken
 * from a fixed array inside the library instead of a caller buffer.
 *   - The array holds MLA_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU the
 *     library runs on, from the first call on that GPU until the process
 *     ends.  A plan whose mla_plan_workspace_bytes exceeds it is refused
 *     with MLA_ERR_WORKSPACE before anything is enqueued.
 *   - Every call uploads the plan's work list into the array (one
 *     host-to-device copy on `stream`, as mla_plan_upload) and then enqueues
 *     the kernels of mla_decode.  No device memory is allocated or freed.
 *   - All calls on one GPU share its array, which keeps the last call's
 *     contents: calls that overlap in time on one GPU (other streams, other
 *     host threads) race on it and must be serialised by the caller.
 * Arguments, results and other errors as for mla_decode.                   */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
mla_status mla_decode_noalloc(const mla_plan* plan, const void* q_nope, const void* q_pe,
                              const void* ckv_cache, const void* kpe_cache, const int32_t* kv_indptr,
                              const int32_t* kv_indices, float sm_scale, void* out, int32_t out_dtype,
                              float* lse, hipStream_t stream);

/* Diagnostics for timing: the next run call made on this host thread has
 * the attention kernel's own dispatch record `before` when the kernel
 * starts and `after` when it ends (hipExtLaunchKernel's start / stop
 * events; the split combine is not included), then forgets both.  Pass
 * NULL, NULL to cancel.  The events are created and owned by the caller;
 * the computation is unchanged.                                           */
mla_status mla_record_attention_events(hipEvent_t before, hipEvent_t after);

/* Static description of a status code. */
const char* mla_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
