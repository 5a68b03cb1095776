// Page-list kernels around the attention kernels (gfx950):
//  * the token-sparse key lists ("Sparse MLA Prefill Kernel": query i
//    attends to the KV rows its index list names; -1 or an index past the
//    end is invalid) are compacted per query token, in order, so that the
//    attention kernel can walk them as page lists of page size 1;
//  * dense block tables ("batch_mla_decode_with_paged_kv_cache" block_tables,
//    FlashMLA block_table) are copied into the CSR page lists of the run calls;
//  * the opt-in checks of a run call's device index arrays (the validate flag
//    of "batch_mla_decode_with_paged_kv_cache": pre-planned runs may skip
//    them) before any attention kernel reads through them.
#include <hip/hip_runtime.h>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kListThreads = 256;
constexpr int kListPerThread = 8;
constexpr int kListChunk = kListThreads * kListPerThread;  // entries per pass

// One workgroup per query token.  A pass loads 2048 entries (8 per thread,
// all loads in flight together), takes one ballot per 256-entry slice, and
// places each valid entry at (entries before its slice) + (valid lanes below
// it in earlier waves and its own wave); one barrier per pass.
__global__ __launch_bounds__(kListThreads) void mla_sparse_lists_kernel(
    const int32_t* __restrict__ indices, int32_t num_tokens, int32_t topk, const int32_t* __restrict__ topk_length,
    int64_t num_slots, int32_t* __restrict__ list, int32_t* __restrict__ count, int32_t* __restrict__ indptr) {
  __shared__ int wave_n[kListPerThread][kListThreads / 64];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = topk_length ? min(max(topk_length[t], 0), topk) : topk;
  const int32_t* src = indices + (size_t)t * topk;
  int32_t* dst = list + (size_t)t * topk;
  const uint64_t below = (1ull << lane) - 1;
  int base = 0;
  for (int c0 = 0; c0 < n; c0 += kListChunk) {
    int32_t v[kListPerThread];
#pragma unroll
    for (int j = 0; j < kListPerThread; ++j) {
      const int k = c0 + j * kListThreads + tid;
      v[j] = k < n ? src[k] : -1;
    }
    uint64_t bal[kListPerThread];
#pragma unroll
    for (int j = 0; j < kListPerThread; ++j) {
      const bool ok = v[j] >= 0 && (int64_t)v[j] < num_slots;  // entries past n hold -1
      bal[j] = __ballot(ok);
      if (lane == 0) wave_n[j][wave] = __popcll(bal[j]);
    }
    __syncthreads();
    int off = base;
#pragma unroll
    for (int j = 0; j < kListPerThread; ++j) {
      int before = 0, total = 0;
#pragma unroll
      for (int w = 0; w < kListThreads / 64; ++w) {
        const int c = wave_n[j][w];
        before += (w < wave) ? c : 0;
        total += c;
      }
      if ((bal[j] >> lane) & 1) dst[off + before + __popcll(bal[j] & below)] = v[j];
      off += total;
    }
    base = off;
    __syncthreads();  // wave_n is rewritten by the next pass
  }
  if (tid == 0) {
    count[t] = base;
    indptr[t] = t * topk;
    if (t == num_tokens - 1) indptr[num_tokens] = num_tokens * topk;
  }
}

// One workgroup per request copies its first kv_indptr[b+1] - kv_indptr[b]
// table entries.
__global__ __launch_bounds__(256) void mla_block_table_kernel(const int32_t* __restrict__ block_table,
                                                              int32_t max_blocks, const int32_t* __restrict__ kv_indptr,
                                                              int32_t* __restrict__ kv_indices) {
  const int b = blockIdx.x;
  const int p0 = kv_indptr[b];
  const int n = min(kv_indptr[b + 1] - p0, max_blocks);
  const int32_t* row = block_table + (size_t)b * max_blocks;
  for (int j = threadIdx.x; j < n; j += 256) kv_indices[p0 + j] = row[j];
}

// One workgroup checks a run call's index arrays against the plan: page
// offsets (start at 0, never decrease, equal to the plan's, or, for capacity
// plans, enough pages for the live key count), query offsets likewise, live
// counts within the plan's bounds, and then, only if all of that holds (so
// the ranges below are the ones the attention kernel would read), every page
// id the run would read lies in [0, num_pages).  Writes the flags found.
__global__ __launch_bounds__(1024) void mla_validate_kernel(ValidateArgs v) {
  __shared__ int flags;
  if (threadIdx.x == 0) flags = 0;
  __syncthreads();
  const bool cap = v.live_kv_len != nullptr;
  int f = 0;
  for (int b = threadIdx.x; b <= v.batch; b += blockDim.x) {
    const int p = v.kv_indptr[b];
    if ((b == 0 && p != 0) || (!cap && p != v.plan_kv_indptr[b])) f |= kValidateIndptr;
    if (v.qo_indptr != nullptr) {
      const int q = v.qo_indptr[b];
      if ((b == 0 && q != 0) || (!cap && q != v.plan_qo_indptr[b])) f |= kValidateQo;
    }
    if (b == v.batch) continue;
    const int pages = v.kv_indptr[b + 1] - p;
    if (pages < 0) f |= kValidateIndptr;
    int n = 1;
    if (v.qo_indptr != nullptr) {
      n = v.qo_indptr[b + 1] - v.qo_indptr[b];
      if (n < 0 || (cap && n > v.max_q)) f |= kValidateQo;
    }
    if (cap) {
      const int L = v.live_kv_len[b];
      if (L < 0 || L > v.max_kv_len) {
        f |= kValidateLengths;
      } else {
        if ((int64_t)pages * v.page_size < L) f |= kValidateIndptr;
        if (v.causal && v.qo_indptr != nullptr && n > L) f |= kValidateLengths;
      }
    }
  }
  if (f) atomicOr(&flags, f);
  __syncthreads();
  if (flags == 0) {
    for (int b = 0; b < v.batch; ++b) {
      const int p0 = v.kv_indptr[b];
      const int need = cap ? (v.live_kv_len[b] + v.page_size - 1) / v.page_size : v.kv_indptr[b + 1] - p0;
      for (int j = threadIdx.x; j < need; j += blockDim.x) {
        const int pg = v.kv_indices[p0 + j];
        if (pg < 0 || pg >= v.num_pages) f |= kValidateIndices;
      }
    }
    if (f) atomicOr(&flags, f);
  }
  __syncthreads();
  if (threadIdx.x == 0) *v.status = flags;
}

}  // namespace

hipError_t launch_validate(const ValidateArgs& v, hipStream_t stream) {
  hipLaunchKernelGGL(mla_validate_kernel, dim3(1), dim3(1024), 0, stream, v);
  return hipGetLastError();
}

hipError_t launch_sparse_lists(const int32_t* indices, int32_t num_tokens, int32_t topk, const int32_t* topk_length,
                               int64_t num_slots, int32_t* list, int32_t* count, int32_t* indptr,
                               hipStream_t stream) {
  if (num_tokens <= 0) return hipSuccess;
  hipLaunchKernelGGL(mla_sparse_lists_kernel, dim3(num_tokens), dim3(kListThreads), 0, stream, indices, num_tokens,
                     topk, topk_length, num_slots, list, count, indptr);
  return hipGetLastError();
}

hipError_t launch_block_table(const int32_t* block_table, int32_t batch, int32_t max_blocks,
                              const int32_t* kv_indptr, int32_t* kv_indices, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(mla_block_table_kernel, dim3(batch), dim3(256), 0, stream, block_table, max_blocks, kv_indptr,
                     kv_indices);
  return hipGetLastError();
}

}  // namespace mla
