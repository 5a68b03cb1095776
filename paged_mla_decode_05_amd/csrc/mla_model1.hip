// MODEL1 record expansion (FlashMLA, "FP8 KV Cache Quantization and
// Dequantization": MODEL1_FP8Sparse has d = 512 for q.k, 448 NoPE dims
// quantised in 7 tiles of 64, 64 RoPE dims).
//
// Record layout (604 bytes per token; the page prints the sizes only, the
// order follows the printed 656-byte layout): bytes 0..447 e4m3 codes of the
// NoPE dims (tile t = dims [64t, 64t+64)), bytes 448..475 seven
// little-endian fp32 scales, bytes 476..603 the 64 RoPE values as bf16.
// The page dequantises to BF16: a NoPE value is bf16(fp32(code) * scale),
// the product in fp32 and the conversion to bf16 both rounding to nearest
// even.
//
// The expansion writes each token as a 576-wide bf16 row in the
// concatenated layout of the attention kernels: dims 0..447 the dequantised
// NoPE values, 448..511 zero, 512..575 the RoPE values.  A query row of 512
// dims (448 + 64) is widened the same way.  With zeros in dims 448..511 of
// both, q.k is the 512-dim product and the first 448 output dims are the
// MODEL1 attention output (V = the 448 NoPE dims); dims 448..511 come out 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kM1Nope = 448;
constexpr int kM1Tile = 64;
constexpr int kM1Record = kM1Nope + 4 * (kM1Nope / kM1Tile) + 2 * kDimKpe;  // 604
constexpr int kRowChunks = (kDimCkv + kDimKpe) / 8;                        // 72 chunks of 8 dims
constexpr int kNopeChunks = kM1Nope / 8;                                   // 56
constexpr int kZeroEnd = kDimCkv / 8;                                      // chunks 56..63 are zero
constexpr int kChunksPerThread = 2;                                        // divides 8 (a tile's chunks)
constexpr int kRowUnits = kRowChunks / kChunksPerThread;
constexpr int kNopeUnits = kNopeChunks / kChunksPerThread;
constexpr int kZeroUnitsEnd = kZeroEnd / kChunksPerThread;
static_assert(8 % kChunksPerThread == 0, "a thread's chunks stay in one tile");
static_assert(kM1Record == 604, "MODEL1 record size");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One e4m3 (OCP "fn") code to its exact fp32 value: bit 7 sign, bits 6..3
// exponent (bias 7), bits 2..0 mantissa; exponent 0 is subnormal
// (m * 2^-9); exponent 15 with mantissa 7 is NaN.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xF, m = c & 7;
  float v = (e == 0) ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  v = (e == 15 && m == 7) ? __builtin_nanf("") : v;
  return (c & 0x80) ? -v : v;
}

// Thread i writes kChunksPerThread consecutive 16-byte chunks (unit i % kRowUnits
// of output row i / kRowUnits); a unit never straddles a 64-dim tile, so one
// scale serves all its codes.  Index math is 32-bit when the unit count fits.
template <typename Index>
__device__ __forceinline__ void model1_record_units(const uint8_t* __restrict__ rec, Index total,
                                                    __bf16* __restrict__ rows) {
  constexpr int K = kChunksPerThread;
  for (Index i = (Index)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (Index)gridDim.x * blockDim.x) {
    const Index t = i / kRowUnits;
    const int c = (int)(i - t * kRowUnits);
    const uint8_t* r = rec + (int64_t)t * kM1Record;
    bf16x8 out[K];
    if (c < kNopeUnits) {
      // 8K codes of tile c * K / 8; the record is 4-byte aligned
      const uint32_t* src = (const uint32_t*)(r + 8 * K * c);
      uint32_t w[2 * K];
#pragma unroll
      for (int j = 0; j < 2 * K; ++j) w[j] = src[j];
      const float scale = *(const float*)(r + kM1Nope + 4 * (c * K / (kM1Tile / 8)));
#pragma unroll
      for (int j = 0; j < K; ++j)
#pragma unroll
        for (int k = 0; k < 8; ++k)
          out[j][k] = (__bf16)(e4m3_value((w[2 * j + (k >> 2)] >> (8 * (k & 3))) & 0xFF) * scale);
    } else if (c < kZeroUnitsEnd) {
#pragma unroll
      for (int j = 0; j < K; ++j) out[j] = bf16x8{};
    } else {
      const uint32_t* src = (const uint32_t*)(r + kM1Nope + 4 * (kM1Nope / kM1Tile) + 16 * K * (c - kZeroUnitsEnd));
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const u32x4 v = {src[4 * j], src[4 * j + 1], src[4 * j + 2], src[4 * j + 3]};
        out[j] = __builtin_bit_cast(bf16x8, v);
      }
    }
    bf16x8* dst = (bf16x8*)(rows + (int64_t)t * (kDimCkv + kDimKpe) + 8 * K * c);
#pragma unroll
    for (int j = 0; j < K; ++j) dst[j] = out[j];
  }
}

__global__ __launch_bounds__(256) void mla_model1_records_kernel(const uint8_t* __restrict__ rec, int64_t n,
                                                                  __bf16* __restrict__ rows) {
  const int64_t total = n * kRowUnits;
  if (total <= INT32_MAX - 65536LL * 256)
    model1_record_units<uint32_t>(rec, (uint32_t)total, rows);
  else
    model1_record_units<int64_t>(rec, total, rows);
}

// Query rows of 512 dims (448 NoPE + 64 RoPE) widened to 576.
__global__ __launch_bounds__(256) void mla_model1_q_kernel(const __bf16* __restrict__ q, int64_t n,
                                                            __bf16* __restrict__ q576) {
  const int64_t total = n * kRowChunks;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / kRowChunks;
    const int c = (int)(i - t * kRowChunks);
    bf16x8 out = bf16x8{};
    if (c < kNopeChunks) {
      out = *(const bf16x8*)(q + t * (kM1Nope + kDimKpe) + 8 * c);
    } else if (c >= kZeroEnd) {
      out = *(const bf16x8*)(q + t * (kM1Nope + kDimKpe) + kM1Nope + 8 * (c - kZeroEnd));
    }
    *(bf16x8*)(q576 + t * (kDimCkv + kDimKpe) + 8 * c) = out;
  }
}

int grid_for(int64_t n, int per_row) {
  const int64_t blocks = (n * per_row + 255) / 256;
  return (int)(blocks < 65536 ? blocks : 65536);  // grid-stride loops cover the rest
}

}  // namespace

hipError_t launch_model1_records(const uint8_t* records, int64_t n, __bf16* rows, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(mla_model1_records_kernel, dim3(grid_for(n, kRowUnits)), dim3(256), 0, stream, records, n, rows);
  return hipGetLastError();
}

hipError_t launch_model1_q(const __bf16* q, int64_t n, __bf16* q576, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(mla_model1_q_kernel, dim3(grid_for(n, kRowChunks)), dim3(256), 0, stream, q, n, q576);
  return hipGetLastError();
}

}  // namespace mla
