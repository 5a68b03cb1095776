// Internal types shared by the host planner / C ABI and the HIP kernels.
#pragma once
#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace mla {

constexpr int kDimCkv = 512;
constexpr int kDimKpe = 64;
constexpr int kFp8RecordBytes = 656;
constexpr int kStageTokens = 64;      // keys per LDS stage; chunk boundaries are multiples
constexpr int kWideRows = 128;        // rows per workgroup in the wide tile mode (4 waves x 32)
constexpr int kNarrowRows = 16;       // rows per workgroup in the narrow tile mode
constexpr int kQuadRowsPerWg = 32;    // rows per workgroup in the quad tile mode
constexpr size_t kWsAlign = 256;

// One workgroup's work: rows [row0, row0+nrows) of request b against keys
// [tok0, tok1).  Rows count (query token, head) pairs of the request as
// token*H + head.  slot < 0: write the final output; else partial slot.
struct WorkItem {
  int32_t b;
  int32_t row0;
  int32_t nrows;
  int32_t tok0;
  int32_t tok1;
  int32_t kv_len;
  int32_t q_len;
  int32_t slot;
};
static_assert(sizeof(WorkItem) == 32, "work item is 8 int32");

// One split (request, row block): its nsplit partial slots are consecutive.
// q_len: query tokens of the request as planned (a capacity plan's bound).
struct SplitGroup {
  int32_t b;
  int32_t row0;
  int32_t nrows;
  int32_t nsplit;
  int32_t slot0;
  int32_t q_len;
  int32_t pad[2];
};
static_assert(sizeof(SplitGroup) == 32, "split group is 8 int32");

struct AttnArgs {
  const void* q_nope;      // bf16 [rows_total, H, 512]
  const void* q_pe;        // bf16 [rows_total, H, 64]
  const void* ckv;         // bf16 [P, ps, 512]   (bf16 format)
  const void* kpe;         // bf16 [P, ps, 64]    (bf16 format)
  const void* kv_fp8;      // u8   [P, ps, 656]   (fp8 format)
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* qo_indptr;  // prefill; nullptr for decode (q row of request b is b)
  const int32_t* wg_ptr;   // [grid+1] item range of each workgroup
  const WorkItem* items;
  const SplitGroup* groups;
  void* out;
  float* lse;
  __bf16* part_o;          // [slots][rows_per_block][512] bf16, normalised partial outputs
  float* part_lse;         // [slots][rows_per_block] fp32 (natural log)
  float scale_log2;        // sm_scale * log2(e)
  int32_t num_heads;
  int32_t page_shift;      // log2(page_size)
  int32_t out_bf16;        // 1: bf16 out, 0: fp32 out
  int32_t causal;          // prefill causal mask
  int32_t rows_per_block;  // partial slot stride in rows
  int32_t num_wgs;         // work lists (one per workgroup, or per sibling group in quad mode)
  int32_t grid;            // workgroups launched
  int32_t group_size;      // quad mode: sibling workgroups per work list
  int32_t xcd_map;         // quad mode: siblings share blockIdx.x mod 8
  int32_t num_items;
  int32_t num_groups;
  int32_t ckv_stride;      // bytes between consecutive token rows of ckv (1024 split, 1152 concatenated)
  int32_t kpe_stride;      // bytes between consecutive token rows of kpe (128 split, 1152 concatenated)
  int32_t q_stride;        // elements between consecutive (token, head) rows of q_nope (512 or 576)
  int32_t qpe_stride;      // elements between consecutive rows of q_pe (64 or 576)
  float out_scale;         // factor applied to the final output rows (1: none)
  // token-sparse decode (all null otherwise): each "request" is one query
  // token whose key list (page size 1) was compacted on the device
  const int32_t* sparse_len;  // [requests] valid keys of each list
  const float* attn_sink;     // [H] sink logit per head (natural-log units), or null
  float* max_logits;          // [rows_total, H] largest logit per row (natural units), or null
  float* part_max;            // [slots][rows_per_block] largest logit of each partial row
  // capacity plans: live key counts [requests] (null otherwise); the plan's
  // items and groups carry the bounds, the kernels clip them to these
  const int32_t* live_kv_len;
  int32_t live_q;             // capacity prefill: live query counts from qo_indptr
  int32_t lse_sq;             // > 0: lse laid out [requests, H, lse_sq]; 0: [rows, H]
};

// Device-array checks of a run call with validate = 1 (mla_lists.hip).
struct ValidateArgs {
  const int32_t* kv_indptr;       // the call's [batch + 1]
  const int32_t* kv_indices;
  const int32_t* qo_indptr;       // prefill; null for decode
  const int32_t* live_kv_len;     // capacity plans; null otherwise
  const int32_t* plan_kv_indptr;  // the plan's copies (in the workspace); null for capacity plans
  const int32_t* plan_qo_indptr;
  int32_t batch, page_size, num_pages, max_kv_len, max_q, causal;
  int32_t* status;                // written: 0 or a set of kValidate* flags
};
constexpr int32_t kValidateIndptr = 1, kValidateIndices = 2, kValidateQo = 4, kValidateLengths = 8;

// Launchers (mla_attn.hip).  They only enqueue on `stream`; return hipError_t.
// t0 / t1: optional events recorded by the attention kernel's own dispatch
// at the start and end of its execution (null: none).
// kv_fp8: 0 bf16 caches, 1 656-byte records, 2 MODEL1 records (604 bytes).
hipError_t launch_attention(const AttnArgs& a, int tile_mode, int kv_fp8, hipStream_t stream, hipEvent_t t0,
                            hipEvent_t t1);
// Decode over fp8 records with an fp8 (e4m3) query: WIDE tile, q_nope =
// the [rows, H, 576] codes with q_stride 576.
hipError_t launch_attention_q8(const AttnArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1);
// Token-sparse attention (WIDE tile, page size 1, key lists bounded by
// a.sparse_len) over fp8 records (a.kv_fp8 set; m1: MODEL1 records) or bf16 rows.
hipError_t launch_sparse_attention(const AttnArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1, bool m1);
// Stable compaction of each query token's key list: entries k < n_t (n_t =
// min(topk_length[t], topk), or topk when topk_length is null) with
// 0 <= idx < num_slots are copied, in order, to list[t * topk ...];
// count[t] = their number; indptr[t] = t * topk (t <= num_tokens).
hipError_t launch_sparse_lists(const int32_t* indices, int32_t num_tokens, int32_t topk,
                               const int32_t* topk_length, int64_t num_slots, int32_t* list, int32_t* count,
                               int32_t* indptr, hipStream_t stream);
hipError_t launch_combine(const AttnArgs& a, hipStream_t stream);
hipError_t launch_validate(const ValidateArgs& v, hipStream_t stream);
// MODEL1 records [n, 604] -> bf16 rows [n, 576]; query rows [n, 512] -> [n, 576].
hipError_t launch_model1_records(const uint8_t* records, int64_t n, __bf16* rows, hipStream_t stream);
hipError_t launch_model1_q(const __bf16* q, int64_t n, __bf16* q576, hipStream_t stream);
// kv_indices[kv_indptr[b] + j] = block_table[b * max_blocks + j] for j < kv_indptr[b+1] - kv_indptr[b].
hipError_t launch_block_table(const int32_t* block_table, int32_t batch, int32_t max_blocks,
                              const int32_t* kv_indptr, int32_t* kv_indices, hipStream_t stream);

}  // namespace mla
