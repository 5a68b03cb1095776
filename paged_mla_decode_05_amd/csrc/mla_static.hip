// Decode without any device allocation: the workspace of mla_decode (work
// list, split partial outputs and their lse) lives in a fixed device array
// of this library instead of a caller buffer, for callers that cannot
// allocate (graph capture, tight serving loops, harnesses that forbid it).
//
// The array is a file-scope __device__ variable: each GPU the library runs
// on holds its own copy, at its own address, until the process ends.  Host
// code never uses the variable's name as a device address (on the host it
// is only a stand-in symbol): the address is looked up once per device with
// hipGetSymbolAddress and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mla.h"
#include "mla_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)MLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// This device's copy of `scratch` (looked up on the first call made on it).
mla_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MLA_ERR_DEVICE;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MLA_OK;
}

}  // namespace

extern "C" mla_status mla_decode_noalloc(const mla_plan* plan, const void* q_nope, const void* q_pe,
                                         const void* ckv_cache, const void* kpe_cache, const int32_t* kv_indptr,
                                         const int32_t* kv_indices, float sm_scale, void* out, int32_t out_dtype,
                                         float* lse, hipStream_t stream) {
  if (!plan) return MLA_ERR_INVALID_ARGUMENT;
  if (mla_plan_workspace_bytes(plan) > kScratchBytes) return MLA_ERR_WORKSPACE;  // before any HIP call
  void* ws = nullptr;
  mla_status st = scratch_for_current_device(&ws);
  if (st != MLA_OK) return st;
  // the plan's work list goes to the head of the array on every call: the
  // previous call on this device may have used another plan
  st = mla_plan_upload(plan, ws, kScratchBytes, stream);
  if (st != MLA_OK) return st;
  return mla_decode(plan, q_nope, q_pe, ckv_cache, kpe_cache, kv_indptr, kv_indices, sm_scale, out, out_dtype, lse,
                    ws, kScratchBytes, stream);
}
