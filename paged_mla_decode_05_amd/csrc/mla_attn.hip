// Paged absorbed-MLA attention kernels for gfx950 (MI355X).
//
// What is computed ("MLA Paged", sections "decode"/"prefill"; FlashMLA
// "Sparse MLA Prefill Kernel" for the lse / exp(P - lse) form; V = the
// first 512 latent dims per "mla_decoding_single_batch"): for every query
// row, logits s_j = sm_scale * (q_nope . ckv_j + q_pe . kpe_j) over the
// keys the row may see, out = softmax(s) @ ckv, lse = ln sum exp(s).
//
// How (our design, for CDNA4):
//  * A persistent grid: workgroup w walks its static list of work items
//    (request, row block, key chunk) made by the host planner.
//  * Gather loader: each 64-key stage is copied HBM -> LDS with 16-byte
//    direct-to-LDS loads (global_load_lds_dwordx4); one wave instruction
//    moves one 1 KB ckv row, or the 128-byte kpe rows of 8 keys.  The page of
//    key T is kv_indices[kv_indptr[b] + (T >> log2 page_size)], slot
//    T & (page_size-1) (FlashMLA's block/offset mapping); keys past the
//    chunk re-read its last live key and are masked, so stale or NaN tail
//    slots are never read.  Two stages are in flight (2 x 72 KB of LDS).
//  * QK^T is computed transposed, S^T = K . Q^T, on bf16 MFMA with the
//    query fragments held in registers; each lane then owns one query row
//    (head), so the online-softmax state (running max m, sum l) is per lane.
//  * P.V is computed as O^T = V^T . P^T: P^T comes straight from the S^T
//    accumulator (no shuffle), V^T from LDS with ds_read_b64_tr_b16.
//  * Online softmax in base 2 on logits pre-scaled by sm_scale*log2(e)
//    (the base-2 trick of FlashMLA's sparse-prefill passage), with a lazy
//    rescale: the running max is only raised when a tile beats it by more
//    than kRescaleSlack, which keeps every P value <= 2^kRescaleSlack.
//  * Tile modes.  WIDE: 4 waves x 32 rows share every key tile
//    (mfma_f32_32x32x16_bf16).  NARROW: one block of 16 rows; the 4 waves
//    split every key tile 16 keys each (mfma_f32_16x16x32_bf16 for S,
//    mfma_f32_16x16x16_bf16 for P.V) and merge their partial results
//    through LDS at the end of the item.
//  * QUAD (selectable): 32 rows per workgroup, waves split keys for S and
//    output dims for P.V; sibling workgroups on one XCD share the key stream
//    through L2.
//  * fp8 656-byte records: raw records to LDS, codes unpacked to exact bf16
//    values, per-tile scales applied in fp32 to the partial logits and to P.
//  * A work item that covers only part of a request's keys writes a
//    normalised partial output and its lse; mla_combine merges them by the
//    log-sum-exp identity (the split-K statistics of
//    "mla_decoding_single_batch").
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kCkvRowBytes = kDimCkv * 2;                      // 1024
constexpr int kKpeRowBytes = kDimKpe * 2;                      // 128
constexpr int kStageCkvBytes = kStageTokens * kCkvRowBytes;    // 65536
constexpr int kStageBytes = kStageCkvBytes + kStageTokens * kKpeRowBytes;  // 73728
constexpr int kLdsBytes = 2 * kStageBytes;                      // 147456
constexpr float kRescaleSlack = 8.0f;                           // log2 units
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.44269504088896341f;

// ---------------------------------------------------------------------------
// LDS layout of one stage: ckv rows [64][1024 B] then kpe rows [64][128 B].
// 16-byte chunks are XOR-swizzled per row so that the MFMA operand reads
// (16 consecutive keys at one chunk; 4 keys x 4 chunks for the transposed
// reads) hit distinct LDS banks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int ckv_swz(int t) {
  const int q = (t >> 2) & 3;
  return ((t & 3) << 2) | (((q & 1) << 1) | (q >> 1));
}
__device__ __forceinline__ int kpe_swz(int t) { return (t >> 1) & 7; }
__device__ __forceinline__ int ckv_off(int t, int c) { return t * kCkvRowBytes + ((c ^ ckv_swz(t)) << 4); }
__device__ __forceinline__ int kpe_off(int t, int c) {
  return kStageCkvBytes + t * kKpeRowBytes + ((c ^ kpe_swz(t)) << 4);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const LDS_AS char* base, int off) {
  return *(const LDS_AS bf16x8*)(base + off);
}

__device__ __forceinline__ i16x4 lds_read_tr(const LDS_AS char* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(base + off));
}

// {x_l, x_(l^32)} for every lane l, through v_permlane32_swap.  The two
// results pass through an empty asm statement: without it the compiler
// treats them as one value (fmaxf(r0, r1) was folded to r0).
__device__ __forceinline__ void xor32_pair(float x, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  uint32_t ra = r[0], rb = r[1];
  asm volatile("" : "+v"(ra), "+v"(rb));
  a = __builtin_bit_cast(float, ra);
  b = __builtin_bit_cast(float, rb);
}
__device__ __forceinline__ float max_xor32(float x) {
  float a, b;
  xor32_pair(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_xor32(float x) {
  float a, b;
  xor32_pair(x, a, b);
  return a + b;
}

// Multiplies an accumulator tile held in AGPRs by alpha through one
// temporary VGPR per element.  Written as asm so that the accumulator keeps
// its AGPR home: a plain C++ multiply makes the register allocator move the
// whole accumulator to VGPRs and spill.
template <int N>
__device__ __forceinline__ void scale_acc(float __attribute__((ext_vector_type(N)))& v, float alpha) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float x = v[i];
    float tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(tmp)
                 : "v"(alpha));
    v[i] = x;
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A compiler memory barrier: LDS reads written after it are not hoisted
// above it, nor those before it sunk below it.  The MFMA loops place one per
// step so that each operand read is issued a fixed number of MFMAs ahead of
// its use (the scheduler would otherwise sink it next to the use); the
// compiler still inserts the lgkmcnt wait before the use.
__device__ __forceinline__ void pin_loads() { asm volatile("" ::: "memory"); }

// S^T chains on mfma_f32_32x32x16_bf16 with the accumulator in VGPRs.  The
// compiler gives every builtin MFMA of these kernels an AGPR accumulator,
// and the 256 AGPRs are O's; S must live in VGPRs, so its MFMAs are written
// here.  The compiler does not see inside the asm, so the hazard distances
// it would insert are written out: each MFMA is preceded by 4 wait states
// (a VALU write of an operand -- converted fp8 codes, a rescaled
// accumulator -- must be that far ahead of the MFMA reading it), which
// overlap the previous MFMA's execution.  mfma32_first starts a chain
// (inline-zero C operand), mfma32_acc continues it (C = D exactly: the
// hardware's back-to-back accumulation), and mfma32_drain puts 24 wait
// states between the last MFMA and the first other reader or writer of the
// accumulator (the XDL write -> VALU read / SrcC read -> VALU write
// distances of gfx950 are shorter).
// kValu = false drops the leading wait states where no operand can have
// been written by a VALU instruction (LDS / global loads only, and C = D).
template <bool kValu = true>
__device__ __forceinline__ void mfma32_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if (kValu) {
    asm volatile("s_nop 3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  } else {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  }
}
template <bool kValu = true>
__device__ __forceinline__ void mfma32_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if (kValu) {
    asm volatile("s_nop 3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
  } else {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
  }
}
// The same for v_mfma_f32_32x32x64_f8f6f4 with e4m3 A and B (32 codes per
// lane: row / column lane % 32, codes 32 (lane / 32) .. +31 of the 64-deep
// step, in byte order) and an fp32 accumulator in VGPRs.  The operands come
// straight from LDS or global loads here, never from a VALU write.
__device__ __forceinline__ void mfma8_first(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma8_acc(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_drain(f32x16& x) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x)); }
__device__ __forceinline__ void mfma32_drain(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}



// Waits until at most `n` vector-memory loads of this wave are outstanding
// (n <= 63); the other counters are left alone.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Direct-to-LDS loads, 16 bytes per lane: lane l reads 16 bytes at
// sbase + voff (or at its own 64-bit address) and writes them to LDS bytes
// [lds + 16 l, lds + 16 l + 16).  The scalar base / 32-bit lane offset form
// keeps the address in one VGPR.  Issued through asm so the compiler neither
// hoists 64-bit per-lane addresses nor inserts waits for them: the caller
// waits with vmcnt and a barrier before any wave reads the destination.  M0
// (the LDS address) and EXEC are saved and restored around the load.
// dma16 / dma16_v with EXEC = {lo, hi} for the load (every lane active at
// the call): zero halves make those lanes move nothing.  Lets a loop issue
// prefetch slices, or a partial slice, without a branch.
__device__ __forceinline__ void dma16_x(const void* sbase, uint32_t voff, uint32_t lds, uint32_t lo, uint32_t hi) {
  uint32_t save;
  uint64_t save_exec;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b64 %1, exec\n\t"
      "s_mov_b32 exec_lo, %5\n\t"
      "s_mov_b32 exec_hi, %6\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b64 exec, %1\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save), "=&s"(save_exec)
      : "v"(voff), "s"(sbase), "s"(lds), "s"(lo), "s"(hi));
}
__device__ __forceinline__ void dma16_vx(const void* vaddr, uint32_t lds, uint32_t lo, uint32_t hi) {
  uint32_t save;
  uint64_t save_exec;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b64 %1, exec\n\t"
      "s_mov_b32 exec_lo, %4\n\t"
      "s_mov_b32 exec_hi, %5\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b64 exec, %1\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save), "=&s"(save_exec)
      : "v"(vaddr), "s"(lds), "s"(lo), "s"(hi));
}
// `on` is wave-uniform; readfirstlane keeps it in an SGPR for the asm operand
// wherever the compiler had moved it to a VGPR.
__device__ __forceinline__ void dma16_on(const void* sbase, uint32_t voff, uint32_t lds, uint32_t on) {
  on = __builtin_amdgcn_readfirstlane(on);
  dma16_x(sbase, voff, lds, on, on);
}
__device__ __forceinline__ void dma16_v_on(const void* vaddr, uint32_t lds, uint32_t on) {
  on = __builtin_amdgcn_readfirstlane(on);
  dma16_vx(vaddr, lds, on, on);
}

// The lane id, re-materialised where it is used: values derived from it are
// cheap to recompute, and keeping them live across the stage loop only
// adds register pressure.
__device__ __forceinline__ int lane_here() {
  int l = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(l));
  return l;
}

__device__ __forceinline__ uint32_t lds_addr(const LDS_AS char* p) { return (uint32_t)(uintptr_t)p; }

// Read-only tables (page indices, work list) are read through the constant
// address space, so uniform reads become scalar loads that do not wait on
// the in-flight direct-to-LDS loads.
#define CONST_AS __attribute__((address_space(4)))
__device__ __forceinline__ int ld_const(const int32_t* p, int i) {
  return ((const CONST_AS int32_t*)p)[i];
}

// Page-size classes of the gather loader (a template parameter, so each
// kernel instantiation has a single addressing path):
//   kPageBig:   page_size >= 64, a 64-key stage lies inside one page;
//   kPageMid:   8 <= page_size < 64, the 8 keys of one kpe load share a page;
//   kPageSmall: page_size < 8.
constexpr int kPageBig = 0, kPageMid = 1, kPageSmall = 2;

// ---------------------------------------------------------------------------
// Gather loader (bf16 caches).  A stage is keys [s_tok0, s_tok0 + 64) of a
// request whose page list starts at kv_indices[page_base]; each wave moves
// 18 slices of it into LDS with 16-byte-per-lane direct loads: slices 0..15
// are the 1 KB ckv rows 16w..16w+15, slices 16..17 the kpe rows of 8 keys
// each.  begin() does the page lookups (scalar loads) and issue(i) one
// slice, so the callers can spread the 18 loads through their MFMA work:
// issued back to back they stall the wave at the address unit.  Every
// address is a uniform (scalar) base plus a 32-bit lane offset.  Keys at or
// past tok_end re-read the chunk's last key (finite data; the softmax masks
// them), so nothing outside the request's live keys is ever read.
// ---------------------------------------------------------------------------
constexpr int kDmaPerWave = 18;

template <int kPageClass>
struct StageLoader {
  const char* ckv_row[16];  // kPageBig: [0] is the stage's first row; else one per ckv slice
  const char* kpe_base[2];
  int kpe_t0[2];            // kPageMid: first (clamped) key of the kpe slice, relative to the stage
  int kpe_page[2];          // kPageSmall: this lane's page
  int last;                 // last live key of the stage, relative to s_tok0
  int s_tok0;
  LDS_AS char* st;
  uint32_t on = ~0u;        // EXEC mask (both halves) of the slices: zero turns issue() into no-ops
  static constexpr int kSlices = kDmaPerWave;

  // page_hint (kPageBig): the stage's page, when the caller looked it up
  // ahead of time (the scalar load then has a whole stage to land).
  __device__ __forceinline__ void begin(const AttnArgs& a, LDS_AS char* stage, int page_base, int tok0,
                                        int tok_end, int wave, int page_hint = -1) {
    const int sh = a.page_shift;
    const int mask = (1 << sh) - 1;
    const char* ckv = (const char*)a.ckv;
    const char* kpe = (const char*)a.kpe;
    st = stage;
    s_tok0 = tok0;
    last = tok_end - 1 - tok0;
    if (kPageClass == kPageBig) {
      const int page = page_hint >= 0 ? page_hint : ld_const(a.kv_indices, page_base + (tok0 >> sh));
      const size_t row0 = ((size_t)page << sh) + (tok0 & mask);
      ckv_row[0] = ckv + row0 * a.ckv_stride;
      kpe_base[0] = kpe + row0 * a.kpe_stride;
      return;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int T = tok0 + min(wave * 16 + i, last);
      const int page = ld_const(a.kv_indices, page_base + (T >> sh));
      ckv_row[i] = ckv + (((size_t)page << sh) + (T & mask)) * a.ckv_stride;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int grp = wave * 2 + i;
      if (kPageClass == kPageMid) {
        // the 8 keys of this slice share one page (clamped keys included)
        const int T0 = tok0 + min(grp * 8, last);
        const int page = ld_const(a.kv_indices, page_base + (T0 >> sh));
        kpe_base[i] = kpe + (((size_t)page << sh) + (T0 & mask)) * a.kpe_stride;
        kpe_t0[i] = T0 - tok0;
      } else {
        // one scalar page lookup per key, then each lane keeps its key's page
        const int lane = lane_here();
        int page = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int Tj = tok0 + min(grp * 8 + j, last);
          const int pj = ld_const(a.kv_indices, page_base + (Tj >> sh));
          page = ((lane >> 3) == j) ? pj : page;
        }
        kpe_page[i] = page;
      }
    }
  }

  __device__ __forceinline__ void issue(const AttnArgs& a, int i, int wave) {
    const int lane = lane_here();
    if (i < 16) {
      const int t = wave * 16 + i;
      const uint32_t swz_off = (uint32_t)((lane ^ ckv_swz(t)) << 4);
      if (kPageClass == kPageBig) {
        dma16_on(ckv_row[0], (uint32_t)(min(t, last) * a.ckv_stride) + swz_off, lds_addr(st + t * kCkvRowBytes), on);
      } else {
        dma16_on(ckv_row[i], swz_off, lds_addr(st + t * kCkvRowBytes), on);
      }
      return;
    }
    const int k = i - 16;
    const int grp = wave * 2 + k;
    const int t = grp * 8 + (lane >> 3);
    const int tc = min(t, last);
    const int c = (lane & 7) ^ kpe_swz(t);
    LDS_AS char* dst = st + kStageCkvBytes + grp * 1024;
    if (kPageClass == kPageBig) {
      dma16_on(kpe_base[0], __umul24((uint32_t)tc, (uint32_t)a.kpe_stride) + (uint32_t)(c << 4), lds_addr(dst), on);
    } else if (kPageClass == kPageMid) {
      dma16_on(kpe_base[k], __umul24((uint32_t)(tc - kpe_t0[k]), (uint32_t)a.kpe_stride) + (uint32_t)(c << 4),
               lds_addr(dst), on);
    } else {
      const int sh = a.page_shift;
      const int T = s_tok0 + tc;
      const char* src = (const char*)a.kpe + (((size_t)kpe_page[k] << sh) + (T & ((1 << sh) - 1))) * a.kpe_stride +
                        (c << 4);
      dma16_v_on(src, lds_addr(dst), on);
    }
  }
};

// The whole stage at once (used where nothing else is in flight).
template <int kPageClass>
__device__ __forceinline__ void issue_stage_bf16(const AttnArgs& a, LDS_AS char* st, int page_base,
                                                 int s_tok0, int tok_end, int wave, int) {
  StageLoader<kPageClass> ld;
  ld.begin(a, st, page_base, s_tok0, tok_end, wave);
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) ld.issue(a, i, wave);
}

// ---------------------------------------------------------------------------
// fp8 record caches (FlashMLA, "FP8 KV Cache Quantization and
// Dequantization"): per token, e4m3 codes of the NoPE dims, one fp32 scale
// per tile of them, and the 64 RoPE dims as bf16.  Two record formats:
//  * FmtV32 (V32_FP8Sparse, 656 bytes): 512 codes, 4 scales of 128-dim
//    tiles, RoPE at byte 528; moved to LDS as it is (41 chunks of 16 bytes).
//  * FmtM1 (MODEL1_FP8Sparse, 604 bytes, packed in the printed order):
//    448 codes, 7 scales of 64-dim tiles at byte 448, RoPE at byte 476.  Its
//    records are 4-byte aligned only, so each one moves as 39 chunks picked
//    per lane that re-lay it in LDS with every field 16-byte aligned:
//    codes at 0..447, RoPE at 448..575, scales 0..3 at 576..591 and 3..6 at
//    592..607 (two overlapping 16-byte reads of the 28 scale bytes), and one
//    pad chunk.  The 624-byte stride (156 dwords, 4 x odd) puts the 16 keys
//    of a K read on distinct LDS banks, as the 164-dword V32 stride does.
// A stage's 64 records sit back to back in LDS at the format's stride.
// Wave w moves the records of keys [16w, 16w+16): lane l of issue i takes
// chunk 64i + l of them.  Keys past tok_end re-read the chunk's last key.
// ---------------------------------------------------------------------------
struct FmtV32 {
  static constexpr bool kM1 = false;
  static constexpr int kRecBytes = kFp8RecordBytes;  // 656 in HBM
  static constexpr int kStride = 656;                // in LDS
  static constexpr int kChunks = 41;
  static constexpr int kNope = 512, kTileDims = 128, kTiles = 4;
  static constexpr int kRopeOff = 528;
  static constexpr bool kPairedDims = true;          // P.V output tiles pair dims D and D + 64
  __device__ static int goff(int c) { return 16 * c; }
  __device__ static int div_chunks(int c) { return (int)(__umul24((uint32_t)c, 200u) >> 13); }  // c / 41, c < 704
  __device__ static int scale_off(int t) { return 512 + 4 * t; }
};
struct FmtM1 {
  static constexpr bool kM1 = true;
  static constexpr int kRecBytes = 604;
  static constexpr int kStride = 624;
  static constexpr int kChunks = 39;
  static constexpr int kNope = 448, kTileDims = 64, kTiles = 7;
  static constexpr int kRopeOff = 448;
  static constexpr bool kPairedDims = false;
  __device__ static int goff(int c) {
    return c < 28 ? 16 * c : (c < 36 ? 476 + 16 * (c - 28) : (c == 36 ? 448 : (c == 37 ? 460 : 0)));
  }
  __device__ static int div_chunks(int c) { return (int)(__umul24((uint32_t)c, 1681u) >> 16); }  // c / 39, c < 640
  __device__ static int scale_off(int t) { return t < 4 ? 576 + 4 * t : 580 + 4 * t; }
  static constexpr int kScaleHiOff = 592;            // the 16-byte chunk holding scales 3 .. 6
};

template <class Fmt>
struct RecLayout {
  static constexpr int kRawBytes = kStageTokens * Fmt::kStride;               // one stage in LDS
  static constexpr int kDmaPerWave = (16 * Fmt::kChunks + 63) / 64;          // 11 (V32), 10 (M1)
  static constexpr int kTail = 16 * Fmt::kChunks - 64 * (kDmaPerWave - 1);   // lanes of the last slice
  static constexpr int kRawOff = kStageBytes;                                 // [bf16 stage][raw 0][raw 1][scales]
  static constexpr int kScaleOff = kStageBytes + 2 * kRawBytes;               // float [tiles][64 keys]
  static constexpr int kNarrowLds = kScaleOff + Fmt::kTiles * kStageTokens * 4;
};
constexpr int kFp8RawBytes = RecLayout<FmtV32>::kRawBytes;                    // 41984
constexpr int kFp8DmaPerWave = RecLayout<FmtV32>::kDmaPerWave;                // 11
constexpr int kFp8LdsBytes = RecLayout<FmtV32>::kNarrowLds;                   // 158720
static_assert(kFp8LdsBytes <= 160 * 1024, "fp8 LDS budget");
static_assert(RecLayout<FmtM1>::kNarrowLds <= kFp8LdsBytes, "MODEL1 records fit the fp8 kernels' LDS");
static_assert(RecLayout<FmtV32>::kTail == 16 && RecLayout<FmtM1>::kTail == 48, "tail slices");

template <int kPageClass, class Fmt = FmtV32>
struct RecordLoader {
  const char* base;  // kPageBig: record of the stage's first key
  int page;          // other classes: lane j < 16 holds the page of key 16w + j (clamped)
  int last;          // last live key of the stage, relative to s_tok0
  int s_tok0;
  LDS_AS char* raw;
  uint32_t on = ~0u;  // EXEC mask (both halves) of the slices: zero turns issue() into no-ops
  static constexpr int kSlices = RecLayout<Fmt>::kDmaPerWave;

  __device__ __forceinline__ void begin(const AttnArgs& a, LDS_AS char* raw_stage, int page_base, int tok0,
                                        int tok_end, int wave) {
    const int sh = a.page_shift;
    const int mask = (1 << sh) - 1;
    raw = raw_stage;
    s_tok0 = tok0;
    last = tok_end - 1 - tok0;
    if (kPageClass == kPageBig) {
      const int pg = ld_const(a.kv_indices, page_base + (tok0 >> sh));
      base = (const char*)a.kv_fp8 + (((size_t)pg << sh) + (tok0 & mask)) * Fmt::kRecBytes;
      return;
    }
    const int lane = lane_here();
    int p = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int T = tok0 + min(wave * 16 + j, last);
      const int pj = ld_const(a.kv_indices, page_base + (T >> sh));
      p = (lane == j) ? pj : p;
    }
    page = p;
  }

  __device__ __forceinline__ void issue(const AttnArgs& a, int i, int wave) {
    const int lane = lane_here();
    const int c = 64 * i + lane;
    const int cc = min(c, 16 * Fmt::kChunks - 1);
    const int tr = Fmt::div_chunks(cc);
    const int k = cc - Fmt::kChunks * tr;
    const int tc = min(wave * 16 + tr, last);
    LDS_AS char* dst = raw + (wave * 16 * Fmt::kChunks + 64 * i) * 16;
    constexpr int kTail = RecLayout<Fmt>::kTail;
    const uint32_t onu = __builtin_amdgcn_readfirstlane(on);  // wave-uniform; keep it scalar for the asm
    const bool tail = i == kSlices - 1;
    uint32_t lo = onu, hi = onu;
    if constexpr (kTail < 32) {
      if (tail) {
        lo = onu & ((1u << kTail) - 1u);
        hi = 0u;
      }
    } else if constexpr (kTail < 64) {
      if (tail) hi = onu & ((1u << (kTail - 32)) - 1u);
    }
    if (kPageClass == kPageBig) {
      dma16_x(base, __umul24((uint32_t)tc, (uint32_t)Fmt::kRecBytes) + (uint32_t)Fmt::goff(k), lds_addr(dst), lo, hi);
    } else {
      const int p = __shfl(page, tr);
      const int sh = a.page_shift;
      const int T = s_tok0 + tc;
      const char* src = (const char*)a.kv_fp8 + (((size_t)p << sh) + (T & ((1 << sh) - 1))) * Fmt::kRecBytes +
                        Fmt::goff(k);
      dma16_vx(src, lds_addr(dst), lo, hi);
    }
  }
};

template <int kPC, class Fmt = FmtV32>
__device__ __forceinline__ void issue_stage_fp8(const AttnArgs& a, LDS_AS char* raw, int page_base, int s_tok0,
                                                int tok_end, int wave) {
  RecordLoader<kPC, Fmt> ld;
  ld.begin(a, raw, page_base, s_tok0, tok_end, wave);
#pragma unroll
  for (int i = 0; i < RecordLoader<kPC, Fmt>::kSlices; ++i) ld.issue(a, i, wave);
}

// Four e4m3 codes (one per byte of x) as bf16, exactly: gfx950's scaled
// OCP fp8 -> bf16 conversion with scale 1 (every e4m3 value - 3 mantissa
// bits, exponents 2^-9 .. 2^8 - is a bf16 value).
__device__ __forceinline__ void codes_to_bf16(uint32_t x, bf16x8& h, int at) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
  h[at + 0] = lo[0];
  h[at + 1] = lo[1];
  h[at + 2] = hi[0];
  h[at + 3] = hi[1];
}

// Wave w unpacks the records of keys [16w, 16w+16) from the raw stage: the
// codes go to the bf16 stage as exact bf16 values (code, not code * scale),
// the rope dims are copied, and the tile scales go to the scale table
// sct[tile][key].  The scale is applied in fp32 by the consumer: to each
// tile's partial dot product in Q.K^T, and to P for the tile's output dims
// in P.V, so no dequantised key is ever rounded.  Lane l handles ckv chunk l
// (dims 8l..8l+7) of every key (MODEL1: lanes 56..63, the dims past the 448
// NoPE dims, write zeros), then two rope chunks; all reads are issued before
// the first conversion.
template <class Fmt = FmtV32>
__device__ __forceinline__ void dequant_stage(const LDS_AS char* __restrict__ raw, LDS_AS char* __restrict__ st,
                                              LDS_AS float* __restrict__ sct, int wave, int lane) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  constexpr int S = Fmt::kStride;
  const bool has = 8 * lane < Fmt::kNope;
  u32x2 codes[16];
  u32x4 rope[2];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    codes[i] = has ? *(const LDS_AS u32x2*)(raw + (wave * 16 + i) * S + 8 * lane) : u32x2{0u, 0u};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = wave * 16 + 8 * i + (lane >> 3);
    rope[i] = *(const LDS_AS u32x4*)(raw + t * S + Fmt::kRopeOff + 16 * (lane & 7));
  }
  // scales: entry e = 64 j + lane < 16 * tiles holds scale e % tiles of key 16w + e / tiles
  constexpr int kScales = 16 * Fmt::kTiles;
  float sc[(kScales + 63) / 64];
#pragma unroll
  for (int j = 0; j < (kScales + 63) / 64; ++j) {
    const int e = min(64 * j + lane, kScales - 1);
    const int key = e / Fmt::kTiles, t = e - Fmt::kTiles * key;
    sc[j] = *(const LDS_AS float*)(raw + (wave * 16 + key) * S + Fmt::scale_off(t));
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    bf16x8 h;
    codes_to_bf16(codes[i][0], h, 0);
    codes_to_bf16(codes[i][1], h, 4);
    *(LDS_AS bf16x8*)(st + ckv_off(wave * 16 + i, lane)) = h;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = wave * 16 + 8 * i + (lane >> 3);
    *(LDS_AS u32x4*)(st + kpe_off(t, lane & 7)) = rope[i];
  }
#pragma unroll
  for (int j = 0; j < (kScales + 63) / 64; ++j) {
    const int e = 64 * j + lane;
    const int key = e / Fmt::kTiles, t = e - Fmt::kTiles * key;
    if (e < kScales) sct[t * kStageTokens + wave * 16 + key] = sc[j];
  }
}

// ---------------------------------------------------------------------------
// Item bookkeeping shared by both modes
// ---------------------------------------------------------------------------
struct RowInfo {
  size_t qrow;  // flattened [total_q * H] index of the row
  int qi;       // query token of the row within its request
  bool ok;      // row exists in this block
};

// Flattened [total_q * H] index of the request's first row: rows r of a
// request (r = query token * H + head) sit at row_base + r.
__device__ __forceinline__ size_t row_base(const AttnArgs& a, const WorkItem& it) {
  const int q_start = a.qo_indptr ? ld_const(a.qo_indptr, it.b) : it.b;
  return (size_t)q_start * a.num_heads;
}

__device__ __forceinline__ RowInfo row_info(const AttnArgs& a, const WorkItem& it, int r_in_block) {
  RowInfo ri;
  const int H = a.num_heads;
  const int r = it.row0 + r_in_block;
  ri.ok = r_in_block < it.nrows;
  const int rr = ri.ok ? r : it.row0;
  ri.qi = rr / H;
  ri.qrow = row_base(a, it) + rr;  // (q_start + qi) * H + head
  return ri;
}

__device__ __forceinline__ int row_key_bound(const AttnArgs& a, const WorkItem& it, const RowInfo& ri) {
  int vis = it.kv_len;
  if (a.causal) vis = it.kv_len - it.q_len + ri.qi + 1;
  if (!ri.ok) vis = 0;
  return min(vis, it.tok1);
}

// Final or partial write of one row's 4 consecutive output dims.
__device__ __forceinline__ void store4(const AttnArgs& a, const WorkItem& it, const RowInfo& ri,
                                       int r_in_block, int dim, f32x4 v) {
  if (it.slot < 0) {
    if (a.out_bf16) {
      bf16x4 h;
      h[0] = (__bf16)v[0];
      h[1] = (__bf16)v[1];
      h[2] = (__bf16)v[2];
      h[3] = (__bf16)v[3];
      *(bf16x4*)((__bf16*)a.out + ri.qrow * kDimCkv + dim) = h;
    } else {
      *(f32x4*)((float*)a.out + ri.qrow * kDimCkv + dim) = v;
    }
  } else {
    bf16x4 h;
    h[0] = (__bf16)v[0];
    h[1] = (__bf16)v[1];
    h[2] = (__bf16)v[2];
    h[3] = (__bf16)v[3];
    *(bf16x4*)(a.part_o + ((size_t)it.slot * a.rows_per_block + r_in_block) * kDimCkv + dim) = h;
  }
}

// Index of a final lse value: row qrow of [rows, H], or, for the layout
// [requests, H, s_q] (FlashMLA's batch x heads x seq_len_q), request b, head
// r % H, query token r / H (r counts the request's rows as token * H + head).
__device__ __forceinline__ size_t lse_index(const AttnArgs& a, int b, int r, size_t qrow) {
  if (a.lse_sq == 0) return qrow;
  const int qi = r / a.num_heads;
  return ((size_t)b * a.num_heads + (r - qi * a.num_heads)) * a.lse_sq + qi;
}

// Capacity plans: the item's rows and key range clipped to this call's live
// counts (a live count above the plan's bound is taken as the bound).  False
// when none of the item's rows exist this call: nothing is computed or
// written for it (the combine skips those rows too).
__device__ __forceinline__ bool clip_live(const AttnArgs& a, WorkItem& it) {
  if (a.live_kv_len == nullptr) return true;
  const int L = min(max(ld_const(a.live_kv_len, it.b), 0), it.kv_len);
  int n = it.q_len;
  if (a.live_q) n = min(max(ld_const(a.qo_indptr, it.b + 1) - ld_const(a.qo_indptr, it.b), 0), it.q_len);
  it.nrows = min(it.nrows, n * a.num_heads - it.row0);
  if (it.nrows <= 0) return false;
  const int vis = a.causal ? L - n + (it.row0 + it.nrows - 1) / a.num_heads + 1 : L;
  it.kv_len = L;
  it.q_len = n;
  it.tok1 = max(it.tok0, min(it.tok1, vis));
  return true;
}

__device__ __forceinline__ void store_lse(const AttnArgs& a, const WorkItem& it, const RowInfo& ri,
                                          int r_in_block, float lse_nat) {
  if (it.slot < 0) {
    a.lse[lse_index(a, it.b, it.row0 + r_in_block, ri.qrow)] = lse_nat;
  } else {
    a.part_lse[(size_t)it.slot * a.rows_per_block + r_in_block] = lse_nat;
  }
}

// ---------------------------------------------------------------------------
// WIDE mode: 4 waves x 32 rows; every wave reads every key of each stage.
//
// LDS addresses are a handful of per-lane base offsets plus compile-time
// immediates: with t = key row and c = 16-byte chunk, the swizzle only
// depends on t mod 16 and only flips the low four bits of c, so stepping c
// by a multiple of 16 (or t by a multiple of 16) is a constant offset.
// ---------------------------------------------------------------------------
struct WideState {
  f32x16 o[16];   // O^T: lane holds row n, dims 32cb + 8(r/4) + 4g + r%4
  float m_run;    // running max (log2 units), per row
  float l_run;    // running sum of this lane's keys
  bool o_live;    // wave-uniform: a P.V has run (before that O is zero and needs no rescale)
  float m_top;    // token-sparse items: the row's largest logit so far (log2 units)
};

// Value fences for hand-interleaving VALU work into an MFMA stream: code
// that uses x runs after hold(x), and x is computed before done(x).  Both
// are empty volatile asm, ordered with the (volatile) MFMA and barrier asm,
// so work placed between them stays in that slot of the instruction stream.
__device__ __forceinline__ void hold(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void done(float x) { asm volatile("" ::"v"(x)); }

// Online-softmax pieces of one 32-key sub-tile S^T (lane: row n, keys
// 8(r/4) + 4g + r%4), split so that they can ride along an MFMA stream.
struct WideSoftmax {
  float mx = kNegInf;
  bool raise = false;
  float alpha = 1.f;
  float mref = 0.f;
};

template <int kPC, bool kPrefetch, bool kSparse = false, class Loader>
__device__ __forceinline__ void wide_stage(const AttnArgs& a, const bf16x8 (&qf)[36], WideState& st,
                                           const LDS_AS char* __restrict__ cur, int stage_tok, int bound,
                                           const int (&kb)[8], const int (&pb)[4], const int (&vb)[8],
                                           int g, Loader& ld, int wave) {
  auto kread = [&](int tb, int ks) -> bf16x8 {
    return ks < 32 ? lds_read_b128(cur, kb[ks & 7] + 256 * (ks >> 3) + tb * kCkvRowBytes)
                   : lds_read_b128(cur, pb[ks - 32] + tb * kKpeRowBytes);
  };
  auto vread = [&](int tb, int j) -> bf16x8 {  // j = 2*cb + kk
    const int cb = j >> 1, kk = j & 1;
    const int imm = (tb + 16 * kk) * kCkvRowBytes + 256 * (cb >> 2);
    const i16x4 v0 = lds_read_tr(cur, vb[cb & 3] + imm);
    const i16x4 v1 = lds_read_tr(cur, vb[4 + (cb & 3)] + imm);
    const i16x8 v = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  // ---- softmax pieces on S^T of sub-tile tb (values scaled to log2 units in place)
  auto sm_scale_mask = [&](float (&sv)[16], WideSoftmax& sm, int tb, int r) {
    float x = sv[r];
    hold(x);
    const int tok = stage_tok + tb + 8 * (r >> 2) + 4 * g + (r & 3);
    x = tok < bound ? x * a.scale_log2 : kNegInf;
    sv[r] = x;
    sm.mx = fmaxf(sm.mx, x);
    done(sm.mx);
  };
  auto sm_decide = [&](WideSoftmax& sm) {  // row max over the sub-tile; raise the running max if needed
    sm.mx = max_xor32(sm.mx);
    if (kSparse) st.m_top = fmaxf(st.m_top, sm.mx);
    sm.raise = __builtin_amdgcn_ballot_w64(sm.mx > st.m_run + kRescaleSlack) != 0;
    if (sm.raise) {
      const float m_new = fmaxf(st.m_run, sm.mx);
      sm.alpha = (st.m_run == kNegInf) ? 0.f : fast_exp2(st.m_run - m_new);
      st.l_run *= sm.alpha;
      st.m_run = m_new;
    }
    sm.mref = (st.m_run == kNegInf) ? 0.f : st.m_run;
    done(sm.mref);
  };
  auto sm_exp = [&](const float (&sv)[16], const WideSoftmax& sm, bf16x8 (&pt)[2], float (&pf)[16], int r) {
    float x = sv[r];
    hold(x);
    const float p = fast_exp2(x - sm.mref);
    st.l_run += p;
    pf[r] = p;
    pt[r >> 3][r & 7] = (__bf16)p;
    done(st.l_run);
  };
  auto rescale_o = [&](float alpha) {
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) scale_acc<16>(st.o[cb], alpha);
  };

  // ---- S^T[32 keys x 32 rows] = K . Q^T over 576 dims for sub-tile tb, with
  // `side(ks)` run after MFMA ks (interleaved VALU work of another phase)
  auto qk = [&](f32x16& sacc, int tb, int dma0, auto&& side) {
    constexpr int KD = 3;  // K fragments in flight
    bf16x8 kr[KD];
#pragma unroll
    for (int i = 0; i < KD; ++i) kr[i] = kread(tb, i);
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      pin_loads();
      if (kPrefetch && (ks & 3) == 0 && dma0 + (ks >> 2) < Loader::kSlices)
        ld.issue(a, dma0 + (ks >> 2), wave);  // up to 9 slices per sub-tile
      const bf16x8 k0 = kr[ks % KD];
      if (ks == 0) {
        mfma32_first<false>(sacc, k0, qf[0]);
      } else {
        mfma32_acc<false>(sacc, k0, qf[ks]);
      }
      if (ks + KD < 36) kr[ks % KD] = kread(tb, ks + KD);
      side(ks);
    }
    pin_loads();
    mfma32_drain(sacc);
  };

  // ---- O^T[32 dims x 32 rows] += V^T[32 dims x 16 keys] . P^T[16 keys x 32 rows] for sub-tile tb.
  // Step i covers dims block cb = i % 16 and keys 16 (i / 16) ..: consecutive
  // MFMAs write different O tiles, so none waits for the one before it.
  auto pv = [&](int tb, bf16x8 (&pt)[2], const float (&pf)[16], auto&& side) {
    constexpr int VD = 3;  // V^T fragments in flight
    auto vstep = [&](int i) { return vread(tb, 2 * (i & 15) + (i >> 4)); };
    bf16x8 vr[VD];
#pragma unroll
    for (int i = 0; i < VD; ++i) vr[i] = vstep(i);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      pin_loads();
      st.o[i & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[i % VD], pt[i >> 4], st.o[i & 15], 0, 0, 0);
      if (i + VD < 32) vr[i % VD] = vstep(i + VD);
      side(i);
    }
    pin_loads();
  };

  // Software pipeline over the two sub-tiles:
  //   QK(0);  QK(1) + softmax(0);  PV(0) + softmax(1);  PV(1)
  // The softmax VALU work issues between MFMAs of the other phase.  A raise
  // of the running max found in softmax(1) rescales O only after PV(0) has
  // accumulated (its P was computed against the old reference).
  f32x16 sa0, sa1;
  float s0[16], s1[16];
  WideSoftmax sm0, sm1;
  bf16x8 pt0[2], pt1[2];
  float pf0[16], pf1[16];
  {
    // Software pipeline over the two sub-tiles:
    //   QK(0);  QK(1) + softmax(0);  PV(0) + softmax(1);  PV(1)
    // The softmax VALU work issues between MFMAs of the other phase.  A
    // raise of the running max found in softmax(1) rescales O only after
    // PV(0) has accumulated (its P was computed against the old reference).
    qk(sa0, 0, 0, [&](int) {});
#pragma unroll
    for (int r = 0; r < 16; ++r) s0[r] = sa0[r];
    qk(sa1, 32, 9, [&](int ks) {
      if (ks < 16) sm_scale_mask(s0, sm0, 0, ks);
      if (ks == 16) sm_decide(sm0);
      if (ks >= 17 && ks < 33) sm_exp(s0, sm0, pt0, pf0, ks - 17);
    });
#pragma unroll
    for (int r = 0; r < 16; ++r) s1[r] = sa1[r];
    if (sm0.raise && st.o_live) rescale_o(sm0.alpha);  // no P.V is in flight here; O is zero until the first P.V
    pv(0, pt0, pf0, [&](int j) {
      if (j < 16) sm_scale_mask(s1, sm1, 32, j);
      if (j == 16) sm_decide(sm1);
      if (j >= 17) sm_exp(s1, sm1, pt1, pf1, j - 17);
    });
    st.o_live = true;
    sm_exp(s1, sm1, pt1, pf1, 15);
    if (sm1.raise) {
      // the last P.V MFMAs write O: let them retire before the AGPRs are read
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
      rescale_o(sm1.alpha);
    }
    pv(32, pt1, pf1, [&](int) {});
  }
}

template <int kPC, bool kSparse = false>
__device__ __forceinline__ void wide_body(const AttnArgs& a, const bf16x8 (&qf)[36], WideState& st,
                                          const LDS_AS char* __restrict__ cur, LDS_AS char* __restrict__ nxt,
                                          bool prefetch, int page_base, int next_tok, int tok_end,
                                          int stage_tok, int bound, const int (&kb)[8], const int (&pb)[4],
                                          const int (&vb)[8], int wave, int lane, int page_hint) {
  // The slices of the next stage ride along this stage's Q.K^T.  For the
  // last stage they are issued with an empty EXEC mask (and addresses of
  // this stage, so every page lookup stays inside the request): one
  // instruction stream, no branch in the MFMA loop.
  StageLoader<kPC> ld;
  ld.begin(a, nxt, page_base, prefetch ? next_tok : stage_tok, tok_end, wave, page_hint);
  ld.on = __builtin_amdgcn_readfirstlane(prefetch ? ~0u : 0u);
  wide_stage<kPC, true, kSparse>(a, qf, st, cur, stage_tok, bound, kb, pb, vb, lane >> 5, ld, wave);
  static_assert(StageLoader<kPC>::kSlices == 18, "two sub-tiles of 9 slices");
}

// WIDE epilogue: lane (n, g) owns row n of the wave's 32 rows, the partner
// lane (n, 1-g) holds the other dims.  bf16 rows (final or partial) are
// staged in LDS and stored whole; fp32 rows are stored in place.
// O^T tile cb, rows 8q + 4g .. +3 (q = 0..3) hold these output dims: 32 cb + 8q + 4g
// in the bf16 tile; in the fp8 tile a tile's upper 16 rows are the dims
// 64 above its lower 16 (the two 16-lane halves of a V^T read then sit on
// disjoint LDS banks), so cb covers dims D + [0, 16) and D + [64, 80) with
// D = 128 (cb / 4) + 16 (cb % 4).
template <bool kPairedDims>
__device__ __forceinline__ int wide_dim(int cb, int q, int g) {
  if (!kPairedDims) return 32 * cb + 8 * q + 4 * g;
  return 128 * (cb >> 2) + 16 * (cb & 3) + (q < 2 ? 8 * q : 64 + 8 * (q - 2)) + 4 * g;
}

// kSparse: token-sparse items also store their largest logit (m_top, log2
// units) and final rows take the attention sink of their head into the
// softmax denominator (one more logit with no value row).
template <bool kPairedDims = false, bool kSparse = false>
__device__ __forceinline__ void wide_epilogue(const AttnArgs& a, const WorkItem& it, WideState& st, const RowInfo& ri,
                                              int rib, LDS_AS char* smem, int wave, int, float m_top = 0.f) {
  const int lane = lane_here();  // recomputed here, not kept (or spilled) across the stage loop
  const int g = lane >> 5;
  const int n = lane & 31;
  const float l_tot = sum_xor32(st.l_run);
  const bool empty = !(l_tot > 0.f);
  float den = l_tot;
  if (kSparse && it.slot < 0 && a.attn_sink != nullptr && !empty) {
    const int head = (it.row0 + rib) % a.num_heads;
    den += fast_exp2(a.attn_sink[head] * kLog2e - st.m_run);
  }
  const float inv = empty ? 0.f : (it.slot < 0 ? a.out_scale : 1.f) / den;  // final rows carry the output scale
  if (ri.ok && g == 0) store_lse(a, it, ri, rib, empty ? kNegInf : (st.m_run + __log2f(l_tot)) * kLn2);
  if (kSparse && ri.ok && g == 0) {
    const float mx = empty ? kNegInf : m_top * kLn2;
    if (it.slot >= 0) {
      a.part_max[(size_t)it.slot * a.rows_per_block + rib] = mx;
    } else if (a.max_logits != nullptr) {
      a.max_logits[ri.qrow] = mx;
    }
  }
  if (a.out_bf16 || it.slot >= 0) {
    // bf16 rows: stage the wave's 32 rows in LDS (free after the loop; 16-byte
    // chunks XOR-swizzled by row), then store each row as one coalesced 1 KB
    LDS_AS char* ob = smem + wave * 32 * kCkvRowBytes;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (__bf16)(st.o[cb][4 * q + e] * inv);
        const int chunk = wide_dim<kPairedDims>(cb, q, 0) >> 3;  // 16-byte chunk of the row
        *(LDS_AS bf16x4*)(ob + n * kCkvRowBytes + ((chunk ^ (n & 7)) << 4) + 8 * g) = h;
      }
    }
    const size_t out_row0 = row_base(a, it) + it.row0 + wave * 32;  // output row of rr = 0
#pragma unroll 4
    for (int rr = 0; rr < 32; ++rr) {
      const u32x4 v = *(const LDS_AS u32x4*)(ob + rr * kCkvRowBytes + ((lane ^ (rr & 7)) << 4));
      if (wave * 32 + rr < it.nrows) {
        __bf16* dst = (it.slot < 0)
                          ? (__bf16*)a.out + (out_row0 + rr) * kDimCkv
                          : a.part_o + ((size_t)it.slot * a.rows_per_block + wave * 32 + rr) * kDimCkv;
        *(u32x4*)(dst + 8 * lane) = v;
      }
    }
    __syncthreads();  // the staging rows overlap the next item's first stage
    return;
  }
  if (ri.ok) {
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {st.o[cb][4 * q] * inv, st.o[cb][4 * q + 1] * inv, st.o[cb][4 * q + 2] * inv,
                         st.o[cb][4 * q + 3] * inv};
        store4(a, it, ri, rib, wide_dim<kPairedDims>(cb, q, g), v);
      }
    }
  }
}

template <int kPC, bool kSparse = false>
__device__ void wide_item(const AttnArgs& a, const WorkItem& it, LDS_AS char* smem, int wave, int) {
  // lane-derived values are recomputed per item: hoisted out of the item
  // loop they would be spilled, and each spill reload waits for every load
  // in flight (the query rows and stage 0)
  const int lane = lane_here();
  const int g = lane >> 5;   // lane half
  const int n = lane & 31;   // row within the wave (S^T / O^T column)
  const int rib = wave * 32 + n;
  const RowInfo ri = row_info(a, it, rib);
  const int bound = row_key_bound(a, it, ri);

  // Stage 0's direct loads go out first, then the query rows: both streams
  // are in flight together and the first stage's wait covers them.  The
  // query loads are unconditional (a missing row reads the item's first row,
  // and its key bound of 0 masks it), so no wait splits them.
  const int page_base = ld_const(a.kv_indptr, it.b);
  const int nstage = (it.tok1 - it.tok0 + kStageTokens - 1) / kStageTokens;
  if (nstage > 0) issue_stage_bf16<kPC>(a, smem, page_base, it.tok0, it.tok1, wave, lane);

  // Query fragments, B operand of S^T = K . Q^T: lane holds row n, dims 8g..8g+7 of each k-step.
  bf16x8 qf[36];
  {
    const __bf16* qn = (const __bf16*)a.q_nope + ri.qrow * a.q_stride + 8 * g;
    const __bf16* qp = (const __bf16*)a.q_pe + ri.qrow * a.qpe_stride + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) qf[ks] = *(const bf16x8*)(qn + 16 * ks);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[32 + ks] = *(const bf16x8*)(qp + 16 * ks);
  }
  // LDS base offsets (see the comment above WideState)
  int kb[8], pb[4], vb[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) kb[k] = ckv_off(n, 2 * k + g);
#pragma unroll
  for (int k = 0; k < 4; ++k) pb[k] = kpe_off(n, 2 * k + g);
  {
    const int t0 = 4 * g + ((lane & 15) >> 2);
    const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int w8 = (lane & 1) ? 8 : 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      vb[k] = ckv_off(t0, 4 * k + cl) + w8;
      vb[4 + k] = ckv_off(t0 + 8, 4 * k + cl) + w8;
    }
  }

  WideState st;
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) st.o[cb] = f32x16{};
  st.m_run = kNegInf;
  st.l_run = 0.f;
  st.o_live = false;
  st.m_top = kNegInf;

  // one-page stages: the page of stage s+1 is looked up a stage ahead (stage 0's when none is next)
  auto page_at = [&](int stage) -> int {
    return kPC == kPageBig ? ld_const(a.kv_indices, page_base + ((it.tok0 + stage * kStageTokens) >> a.page_shift))
                           : -1;
  };
  int pg_next = page_at(nstage > 1 ? 1 : 0);
  for (int s = 0; s < nstage; ++s) {
    const int pg_after = page_at(s + 2 < nstage ? s + 2 : 0);
    wait_vmcnt<0>();
    __syncthreads();
    wide_body<kPC, kSparse>(a, qf, st, smem + (s & 1) * kStageBytes, smem + ((s + 1) & 1) * kStageBytes,
                   s + 1 < nstage, page_base, it.tok0 + (s + 1 < nstage ? s + 1 : 0) * kStageTokens, it.tok1,
                   it.tok0 + s * kStageTokens, bound, kb, pb, vb, wave, lane, pg_next);
    // no barrier here: the buffer of stage s is refilled during stage s + 1,
    // after that stage's top barrier, which every wave passes only once done
    // with stage s
    pg_next = pg_after;
  }
  __syncthreads();  // every wave is done with the last stage before the epilogue stages rows over it
  {
    const int rib_e = wave * 32 + (lane_here() & 31);  // row info recomputed rather than kept across the loop
    wide_epilogue<false, kSparse>(a, it, st, row_info(a, it, rib_e), rib_e, smem, wave, lane, st.m_top);
  }
}

// ---------------------------------------------------------------------------
// WIDE mode with P.V split by output dims (dense bf16 caches).
//
// Q.K^T and the online softmax run as in WIDE: wave w owns query rows
// 32w..32w+31.  P.V is split the other way: wave w accumulates output dims
// 128w..128w+127 of all 128 rows, so each V^T fragment it reads from LDS
// (ds_read_b64_tr_b16, the costly transposed read) feeds four MFMAs, one
// per row block, and a stage's V^T traffic drops from 4 x 64 KB to 64 KB.
// P goes through LDS instead (bf16, 16 KB per stage, plain 16-byte reads),
// with each row's rescale factor.  Per stage:
//   QK(0); QK(1) + softmax(0); publish P0, alpha0; barrier A;
//   rescale; PV(0) + softmax(1); publish P1, alpha1; barrier B; rescale; PV(1)
// P0 has its own 8 KB; P1 goes to the stage's rope rows, which nobody
// reads after barrier A (every wave's Q.K^T of the stage is done).
// O tile 4d + r holds O^T for dims 128w + 32d .., rows 32r ..: lane (n, g)
// is row 32r + n, dims 32d + 8q + 4g + e of the wave's slice (q, e < 4).
// ---------------------------------------------------------------------------
constexpr int kDsPOff = 2 * kStageBytes;                 // P of sub-tile 0: [128 rows][64 B]
constexpr int kDsAlphaOff = kDsPOff + 128 * 64;          // f32 [2 sub-tiles][32 lanes][4 row blocks]
constexpr int kDsLdsBytes = kDsAlphaOff + 2 * 128 * 4;   // 156672
static_assert(kDsLdsBytes <= 160 * 1024, "dim-split LDS budget");
static_assert(kStageBytes - kStageCkvBytes == 128 * 64, "P of sub-tile 1 fills the stage's rope rows");

// Byte offset of lane (n, g)'s 16-byte P^T fragment (k-half kk) of row n of a
// 32-row block in a P buffer: row R holds 4 chunks, chunk 2kk + g being the
// 8 keys that lane (R % 32, g) of the row's owner wave holds for half kk;
// chunks are XOR-swizzled by (R / 2) % 4 so that 8 consecutive rows cover
// 8 distinct 16-byte bank groups.
__device__ __forceinline__ int ds_p_off(int n, int g, int kk) { return n * 64 + 16 * ((2 * kk + g) ^ ((n >> 1) & 3)); }

template <int kPC>
__device__ __forceinline__ void ds_stage(const AttnArgs& a, const bf16x8 (&qf)[36], WideState& st,
                                         LDS_AS char* __restrict__ cur, LDS_AS char* __restrict__ smem,
                                         int stage_tok, int bound, const int (&kb)[8], const int (&pb)[4],
                                         const int (&vb)[8], int g, int n, StageLoader<kPC>& ld, int wave) {
  auto kread = [&](int tb, int ks) -> bf16x8 {
    return ks < 32 ? lds_read_b128(cur, kb[ks & 7] + 256 * (ks >> 3) + tb * kCkvRowBytes)
                   : lds_read_b128(cur, pb[ks - 32] + tb * kKpeRowBytes);
  };
  // V^T fragment: dims block 4 wave + d (32 dims), keys tb + 16 kk .. (16 keys)
  auto vread = [&](int tb, int d, int kk) -> bf16x8 {
    const int off = (tb + 16 * kk) * kCkvRowBytes + 256 * wave;
    const i16x4 v0 = lds_read_tr(cur, vb[d] + off);
    const i16x4 v1 = lds_read_tr(cur, vb[4 + d] + off);
    const i16x8 v = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  auto sm_scale_mask = [&](float (&sv)[16], WideSoftmax& sm, int tb, int r) {
    float x = sv[r];
    hold(x);
    const int tok = stage_tok + tb + 8 * (r >> 2) + 4 * g + (r & 3);
    x = tok < bound ? x * a.scale_log2 : kNegInf;
    sv[r] = x;
    sm.mx = fmaxf(sm.mx, x);
    done(sm.mx);
  };
  auto sm_decide = [&](WideSoftmax& sm) {
    sm.mx = max_xor32(sm.mx);
    sm.raise = __builtin_amdgcn_ballot_w64(sm.mx > st.m_run + kRescaleSlack) != 0;
    sm.alpha = 1.f;
    if (sm.raise) {
      const float m_new = fmaxf(st.m_run, sm.mx);
      sm.alpha = (st.m_run == kNegInf) ? 0.f : fast_exp2(st.m_run - m_new);
      st.l_run *= sm.alpha;
      st.m_run = m_new;
    }
    sm.mref = (st.m_run == kNegInf) ? 0.f : st.m_run;
    done(sm.mref);
  };
  auto sm_exp = [&](const float (&sv)[16], const WideSoftmax& sm, bf16x8 (&pt)[2], int r) {
    float x = sv[r];
    hold(x);
    const float p = fast_exp2(x - sm.mref);
    st.l_run += p;
    pt[r >> 3][r & 7] = (__bf16)p;
    done(st.l_run);
  };

  // The next stage's 18 direct-load slices: one every `dstep` k-steps from
  // slice dma0 up to (not including) dend.
  auto qk = [&](f32x16& sacc, int tb, int dma0, int dstep, int dend, auto&& side) {
    constexpr int KD = 3;  // K fragments in flight
    bf16x8 kr[KD];
#pragma unroll
    for (int i = 0; i < KD; ++i) kr[i] = kread(tb, i);
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      pin_loads();
      if (ks % dstep == 0 && dma0 + ks / dstep < dend) ld.issue(a, dma0 + ks / dstep, wave);
      const bf16x8 k0 = kr[ks % KD];
      if (ks == 0) {
        mfma32_first<false>(sacc, k0, qf[0]);
      } else {
        mfma32_acc<false>(sacc, k0, qf[ks]);
      }
      if (ks + KD < 36) kr[ks % KD] = kread(tb, ks + KD);
      side(ks);
    }
    pin_loads();
    mfma32_drain(sacc);
  };

  // Publish this wave's P (its 32 rows) and rescale factors of a sub-tile.
  auto publish = [&](LDS_AS char* pbuf, const bf16x8 (&pt)[2], const WideSoftmax& sm, int t) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) *(LDS_AS bf16x8*)(pbuf + wave * 2048 + ds_p_off(n, g, kk)) = pt[kk];
    if (g == 0) ((LDS_AS float*)(smem + kDsAlphaOff))[t * 128 + n * 4 + wave] = sm.alpha;
  };
  // After the barrier: scale O rows by their factors when any row of the
  // workgroup raised its running max (the factors are 1 otherwise).
  auto rescale = [&](int t, bool drain) {
    const f32x4 al = *(const LDS_AS f32x4*)(smem + kDsAlphaOff + t * 512 + n * 16);
    const bool any = __builtin_amdgcn_ballot_w64(al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f) != 0;
    if (any && st.o_live) {
      if (drain) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");  // let the last P.V MFMAs retire
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 4; ++r) scale_acc<16>(st.o[4 * d + r], al[r]);
    }
  };
  // O^T[dims of the wave][128 rows] += V^T . P^T over the 32 keys of sub-tile tb.
  // Per k-half: 4 V^T and 4 P^T fragments, 16 MFMAs on 16 different tiles.
  auto pv = [&](int tb, const LDS_AS char* pbuf, auto&& side) {
    bf16x8 va[4], pa[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pa[r] = lds_read_b128(pbuf, r * 2048 + ds_p_off(n, g, 0));
#pragma unroll
    for (int d = 0; d < 4; ++d) va[d] = vread(tb, d, 0);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          pin_loads();
          const int i = 16 * kk + 4 * r + d;
          st.o[4 * d + r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[d], pa[r], st.o[4 * d + r], 0, 0, 0);
          // the other k-half's fragments, each once its last use has issued
          if (kk == 0 && r == 3) va[d] = vread(tb, d, 1);
          if (kk == 0 && d == 3) pa[r] = lds_read_b128(pbuf, r * 2048 + ds_p_off(n, g, 1));
          side(i);
        }
      }
    }
    pin_loads();
  };

  f32x16 sa0, sa1;
  float s0[16], s1[16];
  WideSoftmax sm0, sm1;
  bf16x8 pt0[2], pt1[2];
  LDS_AS char* p0 = smem + kDsPOff;
  LDS_AS char* p1 = cur + kStageCkvBytes;
  // Slices 0-8 ride along Q.K^T of sub-tile 0, 9-13 along sub-tile 1 and
  // 14-17 along the first P.V: issued denser, the loads fill the CU's
  // queue of outstanding misses and the issuing wave stalls in the middle
  // of its MFMA chain; issued during the last P.V they land too late.
  qk(sa0, 0, 0, 4, 9, [&](int) {});
#pragma unroll
  for (int r = 0; r < 16; ++r) s0[r] = sa0[r];
  qk(sa1, 32, 9, 8, 14, [&](int ks) {
    if (ks < 16) sm_scale_mask(s0, sm0, 0, ks);
    if (ks == 16) sm_decide(sm0);
    if (ks >= 17 && ks < 33) sm_exp(s0, sm0, pt0, ks - 17);
  });
#pragma unroll
  for (int r = 0; r < 16; ++r) s1[r] = sa1[r];
  publish(p0, pt0, sm0, 0);
  __syncthreads();  // A: P0 and its factors visible; every wave's Q.K^T of the stage is done
  rescale(0, false);
  pv(0, p0, [&](int i) {
    if (i % 8 == 0) ld.issue(a, 14 + i / 8, wave);
    if (i < 16) sm_scale_mask(s1, sm1, 32, i);
    if (i == 16) sm_decide(sm1);
    if (i >= 17) sm_exp(s1, sm1, pt1, i - 17);
  });
  sm_exp(s1, sm1, pt1, 15);
  st.o_live = true;
  publish(p1, pt1, sm1, 1);
  __syncthreads();  // B: P1 and its factors visible
  rescale(1, true);
  pv(32, p1, [&](int) {});
}

// Dim-split WIDE epilogue: the row owners share 1 / l (and the output scale
// of final rows) through LDS; each wave then writes its 128 dims of every
// row.  bf16 rows are staged in LDS (256 bytes per row slice, 16-byte
// chunks XOR-swizzled by row) and stored 4 rows per instruction.  A lane
// writes 8 bytes (half a chunk); rows R with stage_half(R) = 1 keep their
// two halves swapped, so that the 32 lanes of a write (rows n, n + 8,
// n + 16, n + 24 on the same chunk position) fall on distinct banks; the
// swap is undone on the way out, where it is known at compile time.
__device__ __forceinline__ int stage_half(int R) { return ((R >> 3) ^ (R >> 4)) & 1; }
__device__ __forceinline__ void ds_epilogue(const AttnArgs& a, const WorkItem& it, WideState& st,
                                            LDS_AS char* smem, int wave) {
  const int lane = lane_here();
  const int g = lane >> 5;
  const int n = lane & 31;
  const int rib = wave * 32 + n;
  const RowInfo ri = row_info(a, it, rib);
  const float l_tot = sum_xor32(st.l_run);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : (it.slot < 0 ? a.out_scale : 1.f) / l_tot;
  if (ri.ok && g == 0) store_lse(a, it, ri, rib, empty ? kNegInf : (st.m_run + __log2f(l_tot)) * kLn2);
  LDS_AS float* invb = (LDS_AS float*)(smem + kDsAlphaOff);
  if (g == 0) invb[n * 4 + wave] = inv;
  __syncthreads();
  const f32x4 inv4 = *(const LDS_AS f32x4*)(invb + n * 4);
  if (a.out_bf16 || it.slot >= 0) {
    LDS_AS char* ob = smem + wave * 128 * 256;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int R = 32 * r + n;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x4 h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = (__bf16)(st.o[4 * d + r][4 * q + e] * inv4[r]);
          const int c = 4 * d + q;  // 16-byte chunk of the 256-byte row slice
          *(LDS_AS bf16x4*)(ob + R * 256 + ((c ^ (R & 15)) << 4) + 8 * (g ^ stage_half(R))) = h;
        }
      }
    }
    // every read is issued before the first store: with one wave per SIMD
    // nothing else hides the LDS latency of reads waited for one by one
    const int c = lane & 15;
    u32x4 v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int R = 4 * i + (lane >> 4);
      v[i] = *(const LDS_AS u32x4*)(ob + R * 256 + ((c ^ (R & 15)) << 4));
      if (stage_half(4 * i)) v[i] = u32x4{v[i][2], v[i][3], v[i][0], v[i][1]};  // same for the 4 rows 4i..4i+3
    }
    __bf16* dst = (it.slot < 0 ? (__bf16*)a.out + (row_base(a, it) + it.row0) * kDimCkv
                               : a.part_o + (size_t)it.slot * a.rows_per_block * kDimCkv) +
                  128 * wave + 8 * c;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int R = 4 * i + (lane >> 4);
      if (R < it.nrows) *(u32x4*)(dst + R * kDimCkv) = v[i];
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const RowInfo rr = row_info(a, it, 32 * r + n);
      if (!rr.ok) continue;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = {st.o[4 * d + r][4 * q] * inv4[r], st.o[4 * d + r][4 * q + 1] * inv4[r],
                           st.o[4 * d + r][4 * q + 2] * inv4[r], st.o[4 * d + r][4 * q + 3] * inv4[r]};
          store4(a, it, rr, 32 * r + n, 128 * wave + 32 * d + 8 * q + 4 * g, v);
        }
      }
    }
  }
  __syncthreads();  // the staging rows overlap the next item's first stage
}

template <int kPC>
__device__ void ds_item(const AttnArgs& a, const WorkItem& it, LDS_AS char* smem, int wave) {
  const int lane = lane_here();
  const int g = lane >> 5;
  const int n = lane & 31;
  const RowInfo ri = row_info(a, it, wave * 32 + n);
  const int bound = row_key_bound(a, it, ri);

  // The query rows first (unconditional: a missing row reads the item's
  // first row and is masked by its bound of 0), then stage 0's direct loads,
  // whose page lookups (two dependent scalar loads) the query loads need not
  // wait for.  The first stage waits for both.
  const int page_base = ld_const(a.kv_indptr, it.b);
  const int nstage = (it.tok1 - it.tok0 + kStageTokens - 1) / kStageTokens;
  bf16x8 qf[36];
  {
    const __bf16* qn = (const __bf16*)a.q_nope + ri.qrow * a.q_stride + 8 * g;
    const __bf16* qp = (const __bf16*)a.q_pe + ri.qrow * a.qpe_stride + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) qf[ks] = *(const bf16x8*)(qn + 16 * ks);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[32 + ks] = *(const bf16x8*)(qp + 16 * ks);
  }
  if (nstage > 0) issue_stage_bf16<kPC>(a, smem, page_base, it.tok0, it.tok1, wave, lane);
  int kb[8], pb[4], vb[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) kb[k] = ckv_off(n, 2 * k + g);
#pragma unroll
  for (int k = 0; k < 4; ++k) pb[k] = kpe_off(n, 2 * k + g);
  {
    const int t0 = 4 * g + ((lane & 15) >> 2);
    const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int w8 = (lane & 1) ? 8 : 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      vb[k] = ckv_off(t0, 4 * k + cl) + w8;
      vb[4 + k] = ckv_off(t0 + 8, 4 * k + cl) + w8;
    }
  }

  WideState st;
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) st.o[cb] = f32x16{};
  st.m_run = kNegInf;
  st.l_run = 0.f;
  st.o_live = false;
  st.m_top = kNegInf;

  auto page_at = [&](int stage) -> int {
    return kPC == kPageBig ? ld_const(a.kv_indices, page_base + ((it.tok0 + stage * kStageTokens) >> a.page_shift))
                           : -1;
  };
  int pg_next = page_at(nstage > 1 ? 1 : 0);
  for (int s = 0; s < nstage; ++s) {
    const int pg_after = page_at(s + 2 < nstage ? s + 2 : 0);
    wait_vmcnt<0>();
    __syncthreads();
    LDS_AS char* cur = smem + (s & 1) * kStageBytes;
    StageLoader<kPC> ld;
    const bool more = s + 1 < nstage;
    ld.begin(a, smem + ((s + 1) & 1) * kStageBytes, page_base, it.tok0 + (more ? s + 1 : s) * kStageTokens, it.tok1,
             wave, pg_next);
    ld.on = __builtin_amdgcn_readfirstlane(more ? ~0u : 0u);
    ds_stage<kPC>(a, qf, st, cur, smem, it.tok0 + s * kStageTokens, bound, kb, pb, vb, g, n, ld, wave);
    pg_next = pg_after;
  }
  __syncthreads();  // every wave is done with the last stage before the epilogue uses the LDS
  ds_epilogue(a, it, st, smem, wave);
}

// ---------------------------------------------------------------------------
// WIDE mode over the fp8 record cache, keys dequantised in registers.
//
// The 656-byte records of a stage stay raw in LDS (three stage buffers, the
// loads running two stages ahead); no bf16 copy of the stage is made.
//  * Q.K^T: lane (key n, half h) reads 16 codes, dims 32m + 16h .. +15 of
//    its key, with one ds_read_b128 and converts them exactly to two bf16
//    A fragments (k-steps 2m and 2m+1).  The query fragments follow the same
//    dim order (a permutation inside each 32-dim block), so the product is
//    unchanged.  As in the bf16-staged path, each 128-dim tile's partial dot
//    product is scaled by the key's fp32 tile scale before it is summed.
//  * P.V: the V^T operand (32 dims x 8 keys per lane half) comes from one
//    ds_read_b64_tr_b8 of the raw codes, converted in registers; P is
//    scaled per key by the tile scale of the output dims, as before.
//  * The rope dims are bf16 in the record and are read as they are.
// This halves the LDS bytes per MFMA of the key stream and drops the
// unpack pass; the conversions (one VALU op per 2 codes) issue beside the
// MFMAs.
// ---------------------------------------------------------------------------
constexpr int kW8Bufs = 3;
template <class Fmt>
struct W8Layout {
  static constexpr int kTabOff = kW8Bufs * RecLayout<Fmt>::kRawBytes;                 // per-wave scale tables
  static constexpr int kLdsBytes = kTabOff + 4 * Fmt::kTiles * kStageTokens * 4;      // [4 waves][tiles][64 keys] f32
};
static_assert(W8Layout<FmtV32>::kLdsBytes <= kFp8LdsBytes && W8Layout<FmtM1>::kLdsBytes <= kFp8LdsBytes &&
                  4 * 32 * kCkvRowBytes <= kFp8LdsBytes,
              "fits the fp8 kernels' LDS");

__device__ __forceinline__ bf16x8 codes8(uint32_t lo, uint32_t hi) {
  bf16x8 h;
  codes_to_bf16(lo, h, 0);
  codes_to_bf16(hi, h, 4);
  return h;
}

// kQ8: the query is e4m3 codes too ([rows, H, 576] bytes, no scale: the
// fp8 query type of "mla_decoding_single_batch").  Q.K^T over the 512
// latent dims then runs on the fp8 x fp8 MFMA (32x32x64), 64 dims per step,
// straight from the key codes in LDS (no conversion); the 64 rope dims are
// converted to bf16 once (exactly) and stay on the bf16 MFMA, as does P.V.
// Fmt: the record format (FmtV32 or FmtM1; kQ8 with FmtV32 only).  MODEL1
// records have 448 NoPE dims in 7 tiles of 64: 14 code steps of 32 dims in
// Q.K^T, folded every 2 steps, and 14 output tiles of 32 dims in P.V (tiles
// 14 and 15, dims 448..511, stay 0); their output tiles hold 32 consecutive
// dims, so each one lies inside one scale tile.
template <int kPC, bool kSparse = false, bool kQ8 = false, class Fmt = FmtV32>
__device__ void wide8_item(const AttnArgs& a, const WorkItem& it, LDS_AS char* smem, int wave, int) {
  static_assert(!kQ8 || !Fmt::kM1, "the e4m3 query runs over the 656-byte records");
  constexpr int S = Fmt::kStride;                 // record stride in LDS
  constexpr int kRaw = RecLayout<Fmt>::kRawBytes; // one stage
  constexpr int kDma = RecLayout<Fmt>::kDmaPerWave;
  constexpr int kM = Fmt::kNope / 32;             // 32-dim code steps of Q.K^T
  constexpr int kMT = Fmt::kTileDims / 32;        // code steps per scale tile
  constexpr int kT = Fmt::kTiles;
  constexpr int kJ = 2 * kM;                      // P.V steps (32 output dims x 16 keys each)
  const int lane = lane_here();  // lane-derived values recomputed per item (kept across items they get spilled)
  const int g = lane >> 5;
  const int n = lane & 31;
  const int rib = wave * 32 + n;
  const RowInfo ri = row_info(a, it, rib);
  const int bound = row_key_bound(a, it, ri);

  // Stage 0's records go out first, then the query rows, then stage 1: the
  // first stage's wait (all but one stage's loads) then covers the query.
  // The query loads are unconditional (a missing row reads the item's first
  // row and is masked by its key bound of 0), so no wait splits them.
  const int page_base = ld_const(a.kv_indptr, it.b);
  const int nstage = (it.tok1 - it.tok0 + kStageTokens - 1) / kStageTokens;
  if (nstage > 0) issue_stage_fp8<kPC, Fmt>(a, smem, page_base, it.tok0, it.tok1, wave);

  // Query fragments in the codes' dim order: nope k-step 2m+s, half g holds
  // dims 32m + 16g + 8s .. +7; rope k-steps as in the bf16 path.  kQ8: step
  // c of the fp8 MFMA, half g holds the codes of dims 64c + 32g .. +31.
  bf16x8 qf[kQ8 ? 1 : 2 * kM];
  bf16x8 qr[4];
  i32x8 q8[kQ8 ? 8 : 1];
  if constexpr (kQ8) {
    const uint8_t* qc = (const uint8_t*)a.q_nope + ri.qrow * a.q_stride;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u32x4 lo = *(const u32x4*)(qc + 64 * c + 32 * g);
      const u32x4 hi = *(const u32x4*)(qc + 64 * c + 32 * g + 16);
      q8[c] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 c8 = *(const u32x2*)(qc + kDimCkv + 16 * ks + 8 * g);
      qr[ks] = codes8(c8[0], c8[1]);
    }
  } else {
    const __bf16* qn = (const __bf16*)a.q_nope + ri.qrow * a.q_stride + 16 * g;
    const __bf16* qp = (const __bf16*)a.q_pe + ri.qrow * a.qpe_stride + 8 * g;
#pragma unroll
    for (int m = 0; m < kM; ++m)
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) qf[2 * m + sh] = *(const bf16x8*)(qn + 32 * m + 8 * sh);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qr[ks] = *(const bf16x8*)(qp + 16 * ks);
  }
  // byte offsets inside a raw stage
  const int kaddr = n * S + (kQ8 ? 32 : 16) * g;           // + tb*S + 32m (kQ8: + 64c)
  const int raddr = n * S + Fmt::kRopeOff + 16 * g;        // rope: + tb*S + 32kr
  int vaddr;
  {
    // tr_b8: in each 16-lane group, lane pair j supplies key 8(j/4) + 4h + j%4
    // of the 16-key step (h = lane / 32), dims P((lane/16)%2) + 8(lane%2) ..
    // of the output tile: P = 64 for V32's paired dims, 16 for MODEL1's
    // consecutive ones (see wide_dim)
    const int p = lane & 15, j = p >> 1;
    const int vkey = 8 * (j >> 2) + 4 * g + (j & 3);
    vaddr = vkey * S + (Fmt::kPairedDims ? 64 : 16) * ((lane >> 4) & 1) + 8 * (p & 1);  // + (tb + 16kk)*S + D(cb)
  }
  LDS_AS float* tab = (LDS_AS float*)(smem + W8Layout<Fmt>::kTabOff) + wave * kT * kStageTokens;

  WideState st;
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) st.o[cb] = f32x16{};
  st.m_run = kNegInf;
  st.l_run = 0.f;
  st.o_live = false;
  float m_top = kNegInf;  // token-sparse: the row's largest logit (log2 units)

  if (nstage > 1) issue_stage_fp8<kPC, Fmt>(a, smem + kRaw, page_base, it.tok0 + kStageTokens, it.tok1, wave);
  for (int s = 0; s < nstage; ++s) {
    // stage s must have landed; stage s+1's records may still be in flight
    if (s + 1 < nstage) {
      wait_vmcnt<kDma>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();  // stage s visible; every wave is done with stage s-1 (its buffer is refilled below)
    const int buf = s % kW8Bufs;
    const LDS_AS char* __restrict__ raw = smem + buf * kRaw;
    // this lane's K codes and V^T rows: the sums are kept in registers (the
    // empty asm makes them opaque), so every read below is base + immediate
    uint32_t kb_u = lds_addr(raw) + kaddr, vb_u = lds_addr(raw) + vaddr, rb_u = lds_addr(raw) + raddr;
    asm volatile("" : "+v"(kb_u), "+v"(vb_u), "+v"(rb_u));
    const LDS_AS char* __restrict__ kbase = (const LDS_AS char*)(uintptr_t)kb_u;
    const LDS_AS char* __restrict__ vbase = (const LDS_AS char*)(uintptr_t)vb_u;
    const LDS_AS char* __restrict__ rbase = (const LDS_AS char*)(uintptr_t)rb_u;  // rope dims
    const bool more = s + 2 < nstage;
    RecordLoader<kPC, Fmt> ld;
    ld.begin(a, smem + ((s + 2) % kW8Bufs) * kRaw, page_base, it.tok0 + (more ? s + 2 : s) * kStageTokens,
             it.tok1, wave);
    ld.on = __builtin_amdgcn_readfirstlane(more ? ~0u : 0u);
    {
      // this wave's copy of the stage's tile scales: tab[t][key]
      const f32x4 sc = *(const LDS_AS f32x4*)(raw + lane * S + Fmt::scale_off(0));
#pragma unroll
      for (int t = 0; t < 4; ++t) tab[t * kStageTokens + lane] = sc[t];
      if constexpr (kT > 4) {
        const f32x4 sc2 = *(const LDS_AS f32x4*)(raw + lane * S + FmtM1::kScaleHiOff);  // scales 3 .. 6
#pragma unroll
        for (int t = 4; t < kT; ++t) tab[t * kStageTokens + lane] = sc2[t - 3];
      }
    }
    const int stage_tok = it.tok0 + s * kStageTokens;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int tb = sub * 32;
      auto scales = [&](int t, int q) -> f32x4 {
        return *(const LDS_AS f32x4*)(tab + t * kStageTokens + tb + 8 * q + 4 * g);
      };
      // ---- S^T[32 keys x 32 rows]: the rope chain starts the accumulator,
      // then each 128-dim tile t runs its own chain into part[t % 2]; its
      // per-key scaling into sacc is issued two steps into the next tile's
      // chain, so the VALU work and its wait states overlap MFMAs.
      f32x16 sacc, part[2];
      {
        bf16x8 rp[4];  // all four rope fragments in flight before the chain starts
#pragma unroll
        for (int kr2 = 0; kr2 < 4; ++kr2) rp[kr2] = *(const LDS_AS bf16x8*)(rbase + tb * S + 32 * kr2);
        pin_loads();
#pragma unroll
        for (int kr2 = 0; kr2 < 4; ++kr2) {
          if (kr2 == 0) {
            mfma32_first<false>(sacc, rp[0], qr[0]);
          } else {
            mfma32_acc<false>(sacc, rp[kr2], qr[kr2]);
          }
        }
      }
      f32x4 tsc[4];  // the scales of the lane's keys in the tile being folded in
      auto fold = [&](int t) {  // sacc += part[t % 2] * (tile t's key scales)
        mfma32_drain(part[t & 1], sacc);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int r = 0; r < 4; ++r) sacc[4 * q + r] += part[t & 1][4 * q + r] * tsc[q][r];
      };
      if constexpr (kQ8) {
        // two 64-deep fp8 steps per 128-dim tile
        constexpr int KD8 = 2;  // 32-code reads in flight
        auto kread8 = [&](int c) -> i32x8 {
          const u32x4 lo = *(const LDS_AS u32x4*)(kbase + tb * S + 64 * c);
          const u32x4 hi = *(const LDS_AS u32x4*)(kbase + tb * S + 64 * c + 16);
          return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        };
        i32x8 kr8[KD8];
#pragma unroll
        for (int i = 0; i < KD8; ++i) kr8[i] = kread8(i);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          pin_loads();
          const i32x8 kc = kr8[c % KD8];
          if (c + KD8 < 8) kr8[c % KD8] = kread8(c + KD8);
          f32x16& pa = part[(c >> 1) & 1];
          if ((c & 1) == 0) {
            mfma8_first(pa, kc, q8[c]);
          } else {
            mfma8_acc(pa, kc, q8[c]);
          }
          if ((c & 1) == 0 && c > 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) tsc[q] = scales((c >> 1) - 1, q);
          }
          if ((c & 1) == 1 && c > 1) fold((c >> 1) - 1);
        }
      } else {
      constexpr int KD = 3;  // 16-code reads in flight
      u32x4 kr[KD];
      auto kread = [&](int m) -> u32x4 { return *(const LDS_AS u32x4*)(kbase + tb * S + 32 * m); };
#pragma unroll
      for (int i = 0; i < KD; ++i) kr[i] = kread(i);
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        pin_loads();
        const u32x4 c = kr[m % KD];
        if (m + KD < kM) kr[m % KD] = kread(m + KD);
        const bf16x8 a0 = codes8(c[0], c[1]), a1 = codes8(c[2], c[3]);
        f32x16& pa = part[(m / kMT) & 1];
        if (m % kMT == 0) {
          mfma32_first(pa, a0, qf[2 * m]);
        } else {
          mfma32_acc(pa, a0, qf[2 * m]);
        }
        mfma32_acc(pa, a1, qf[2 * m + 1]);
        if (m % kMT == 0 && m > 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) tsc[q] = scales(m / kMT - 1, q);
        }
        if (m % kMT == 1 && m > 1) fold(m / kMT - 1);
      }
      }
      pin_loads();
#pragma unroll
      for (int q = 0; q < 4; ++q) tsc[q] = scales(kT - 1, q);
      fold(kT - 1);
      // ---- online softmax (base 2); lane holds keys 8(r/4) + 4g + r%4 of the sub-tile
      float sv[16];
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = stage_tok + tb + 8 * (r >> 2) + 4 * g + (r & 3);
        const float x = sacc[r] * a.scale_log2;
        sv[r] = tok < bound ? x : kNegInf;
        mx = fmaxf(mx, sv[r]);
      }
      mx = max_xor32(mx);
      if (kSparse) m_top = fmaxf(m_top, mx);
      if (__builtin_amdgcn_ballot_w64(mx > st.m_run + kRescaleSlack) != 0) {
        const float m_new = fmaxf(st.m_run, mx);
        const float alpha = (st.m_run == kNegInf) ? 0.f : fast_exp2(st.m_run - m_new);
        st.l_run *= alpha;
        if (__builtin_amdgcn_ballot_w64(st.m_run != kNegInf) != 0) {  // else O is still zero
#pragma unroll
          for (int cb = 0; cb < 16; ++cb) scale_acc<16>(st.o[cb], alpha);
        }
        st.m_run = m_new;
      }
      const float mref = (st.m_run == kNegInf) ? 0.f : st.m_run;
      float pf[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pf[r] = fast_exp2(sv[r] - mref);
        st.l_run += pf[r];
      }
      // ---- O^T[32 dims x 32 rows] += V^T[32 dims x 16 keys] . P^T[16 keys x 32 rows]
      constexpr int VD = 3;
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      typedef int i32x2 __attribute__((ext_vector_type(2)));
      auto vread = [&](int j) -> u32x2 {  // j = 2*cb + kk
        const int cb = j >> 1, kk = j & 1;
        const int dcol = Fmt::kPairedDims ? 128 * (cb >> 2) + 16 * (cb & 3) : 32 * cb;
        const LDS_AS char* src = vbase + (tb + 16 * kk) * S + dcol;
        return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)src));
      };
      u32x2 vr[VD];
#pragma unroll
      for (int i = 0; i < VD; ++i) vr[i] = vread(i);
      bf16x8 pt[2];
      f32x4 nsc[4];  // scales of the next tile, read half a tile ahead
#pragma unroll
      for (int q = 0; q < 4; ++q) nsc[q] = scales(0, q);
      constexpr int kJT = 2 * kMT;  // P.V steps per scale tile
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        pin_loads();
        if (j % kJT == 0) {
          // output dims of tile j / kJT: P scaled by each key's tile scale
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) pt[q >> 1][4 * (q & 1) + r] = (__bf16)(pf[4 * q + r] * nsc[q][r]);
        }
        if (j % kJT == kJT / 2 && j < kJ - kJT) {
#pragma unroll
          for (int q = 0; q < 4; ++q) nsc[q] = scales(j / kJT + 1, q);
        }
        const u32x2 v = vr[j % VD];
        if (j + VD < kJ) vr[j % VD] = vread(j + VD);
        st.o[j >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(codes8(v[0], v[1]), pt[j & 1], st.o[j >> 1], 0, 0, 0);
        // the records of the stage after next ride along P.V (Q.K^T waits on its own LDS reads)
        if ((j & 3) == 0 && sub * (kJ / 4) + (j >> 2) < RecordLoader<kPC, Fmt>::kSlices)
          ld.issue(a, sub * (kJ / 4) + (j >> 2), wave);
      }
      pin_loads();
    }
  }
  __syncthreads();  // every wave is done with the stage buffers before the epilogue stages rows there
  {
    const int rib_e = wave * 32 + (lane_here() & 31);  // row info recomputed rather than kept across the loop
    wide_epilogue<Fmt::kPairedDims, kSparse>(a, it, st, row_info(a, it, rib_e), rib_e, smem, wave, lane, m_top);
  }
}

// ---------------------------------------------------------------------------
// NARROW mode: one block of <= 16 rows; wave w takes keys [16w, 16w+16) of
// each stage; the four partial results are merged through LDS.
// ---------------------------------------------------------------------------
constexpr int kMergeRowFloats = kDimCkv + 4;  // padded row of the merge buffer

struct NarrowState {
  f32x4 o[32];    // O^T: lane holds row n, dims 16cb + 4g4 + r
  float m_run;
  float l_run;
};

// kM1 (fp8 only): MODEL1 records, 448 NoPE dims in 64-dim scale tiles; the
// k-steps and output tiles past dim 448 are skipped (their keys are zero).
template <int kPC, bool kFp8, bool kM1 = false>
__device__ __forceinline__ void narrow_body(const AttnArgs& a, const bf16x8 (&qf)[18], NarrowState& st,
                                            const LDS_AS char* __restrict__ cur, LDS_AS char* __restrict__ nxt,
                                            bool prefetch, int page_base, int next_tok, int tok_end,
                                            int stage_tok, int bound, const int (&kb)[4], const int (&pb)[2],
                                            const int (&vb)[8], int wave, int lane,
                                            const LDS_AS float* __restrict__ sct) {
  StageLoader<kPC> ld;
  if (prefetch) ld.begin(a, nxt, page_base, next_tok, tok_end, wave);
  const int g4 = lane >> 4;
  const int tb = wave * 16;
  // fp8 cache: scales of this lane's keys tb + 4 g4 + (0..3) in tile t
  auto scales = [&](int t) -> f32x4 { return *(const LDS_AS f32x4*)(sct + t * kStageTokens + tb + 4 * g4); };
  // S^T[16 keys x 16 rows]
  f32x4 sacc = {};
  f32x4 part = {};
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) {
    if (prefetch) ld.issue(a, ks, wave);  // one prefetch slice per k-step
    if (kM1 && (ks == 14 || ks == 15)) continue;  // dims 448..511
    const bf16x8 kf = ks < 16 ? lds_read_b128(cur, kb[ks & 3] + 256 * (ks >> 2)) : lds_read_b128(cur, pb[ks - 16]);
    if (kFp8 && ks < 16) {
      constexpr int kKsPerTile = kM1 ? 2 : 4;  // 32-dim k-steps per scale tile
      part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], part, 0, 0, 0);
      if (ks % kKsPerTile == kKsPerTile - 1) {
        sacc += part * scales(ks / kKsPerTile);
        part = f32x4{};
      }
    } else {
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], sacc, 0, 0, 0);
    }
  }
  float sv[4];
  float mx = kNegInf;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tok = stage_tok + tb + 4 * g4 + r;
    const float x = sacc[r] * a.scale_log2;
    sv[r] = tok < bound ? x : kNegInf;
    mx = fmaxf(mx, sv[r]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const bool need = mx > st.m_run + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = (st.m_run == kNegInf) ? 0.f : fast_exp2(st.m_run - m_new);
    st.l_run *= alpha;
    if (__builtin_amdgcn_ballot_w64(st.m_run != kNegInf) != 0) {  // else O is still zero
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) {
        st.o[cb] *= alpha;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    st.m_run = m_new;
  }
  const float mref = (st.m_run == kNegInf) ? 0.f : st.m_run;
  i16x4 pt;
  f32x4 pf;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float p = fast_exp2(sv[r] - mref);
    st.l_run += p;
    pf[r] = p;
    pt[r] = __builtin_bit_cast(short, (__bf16)p);
  }
  // O^T[16 dims x 16 rows] += V^T[16 dims x 16 keys] . P^T[16 keys x 16 rows]
#pragma unroll
  for (int cb = 0; cb < (kM1 ? 28 : 32); ++cb) {
    constexpr int kCbPerTile = kM1 ? 4 : 8;  // 16-dim output tiles per scale tile
    if (kFp8 && cb % kCbPerTile == 0) {
      // output dims of tile cb / kCbPerTile: P scaled by each key's tile scale
      const f32x4 ps = pf * scales(cb / kCbPerTile);
#pragma unroll
      for (int r = 0; r < 4; ++r) pt[r] = __builtin_bit_cast(short, (__bf16)ps[r]);
    }
    const i16x4 v = lds_read_tr(cur, vb[cb & 7] + 256 * (cb >> 3));
    st.o[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, pt, st.o[cb], 0, 0, 0);
  }
}

template <int kPC, bool kFp8, bool kM1 = false>
__device__ void narrow_item(const AttnArgs& a, const WorkItem& it, LDS_AS char* smem, int wave, int lane) {
  using Fmt = typename std::conditional<kM1, FmtM1, FmtV32>::type;
  using RL = RecLayout<Fmt>;
  const int g4 = lane >> 4;  // lane quarter
  const int n = lane & 15;   // row within the block
  const RowInfo ri = row_info(a, it, n);
  const int bound = row_key_bound(a, it, ri);

  bf16x8 qf[18];
  {
    const bf16x8 z = {};
    const __bf16* qn = (const __bf16*)a.q_nope + ri.qrow * a.q_stride + 8 * g4;
    const __bf16* qp = (const __bf16*)a.q_pe + ri.qrow * a.qpe_stride + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = ri.ok && 32 * ks < (kM1 ? FmtM1::kNope : kDimCkv) ? *(const bf16x8*)(qn + 32 * ks) : z;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qf[16 + ks] = ri.ok ? *(const bf16x8*)(qp + 32 * ks) : z;
  }
  int kb[4], pb[2], vb[8];
  {
    const int t = wave * 16 + n;
#pragma unroll
    for (int k = 0; k < 4; ++k) kb[k] = ckv_off(t, 4 * k + g4);
#pragma unroll
    for (int k = 0; k < 2; ++k) pb[k] = kpe_off(t, 4 * k + g4);
    const int t0 = wave * 16 + 4 * g4 + ((lane & 15) >> 2);
    const int x = (lane & 3) >> 1;
    const int w8 = (lane & 1) ? 8 : 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) vb[k] = ckv_off(t0, 2 * k + x) + w8;
  }

  NarrowState st;
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) st.o[cb] = f32x4{};
  st.m_run = kNegInf;
  st.l_run = 0.f;

  const int page_base = ld_const(a.kv_indptr, it.b);
  const int nstage = (it.tok1 - it.tok0 + kStageTokens - 1) / kStageTokens;
  if (kFp8) {
    LDS_AS char* raw = smem + RL::kRawOff;
    LDS_AS float* sct = (LDS_AS float*)(smem + RL::kScaleOff);
    if (nstage > 0) issue_stage_fp8<kPC, Fmt>(a, raw, page_base, it.tok0, it.tok1, wave);
    if (nstage > 1) issue_stage_fp8<kPC, Fmt>(a, raw + RL::kRawBytes, page_base, it.tok0 + kStageTokens, it.tok1, wave);
    for (int s = 0; s < nstage; ++s) {
      if (s + 1 < nstage) {
        wait_vmcnt<RL::kDmaPerWave>();
      } else {
        wait_vmcnt<0>();
      }
      __syncthreads();
      dequant_stage<Fmt>(raw + (s & 1) * RL::kRawBytes, smem, sct, wave, lane);
      __syncthreads();
      if (s + 2 < nstage)
        issue_stage_fp8<kPC, Fmt>(a, raw + (s & 1) * RL::kRawBytes, page_base, it.tok0 + (s + 2) * kStageTokens,
                                  it.tok1, wave);
      narrow_body<kPC, true, kM1>(a, qf, st, smem, smem, false, page_base, 0, it.tok1, it.tok0 + s * kStageTokens,
                                  bound, kb, pb, vb, wave, lane, sct);
    }
    __syncthreads();
  } else {
    if (nstage > 0) issue_stage_bf16<kPC>(a, smem, page_base, it.tok0, it.tok1, wave, lane);
    for (int s = 0; s < nstage; ++s) {
      wait_vmcnt<0>();
      __syncthreads();
      narrow_body<kPC, false>(a, qf, st, smem + (s & 1) * kStageBytes, smem + ((s + 1) & 1) * kStageBytes,
                       s + 1 < nstage, page_base, it.tok0 + (s + 1) * kStageTokens, it.tok1,
                       it.tok0 + s * kStageTokens, bound, kb, pb, vb, wave, lane, nullptr);
      // stage s's buffer is refilled during stage s + 1, after its top barrier
    }
    __syncthreads();  // every wave is done with the last stage before the merge buffer is written
  }

  // ---- merge the four waves' partial results through LDS ----
  float l_run = st.l_run;
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  LDS_AS float* mbuf = (LDS_AS float*)smem;                       // [4][16][kMergeRowFloats]
  LDS_AS float* stats = mbuf + 4 * 16 * kMergeRowFloats;         // [4][16][2]
  if (g4 == 0) {
    stats[(wave * 16 + n) * 2 + 0] = st.m_run;
    stats[(wave * 16 + n) * 2 + 1] = l_run;
  }
  __syncthreads();
  float m_all = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) m_all = fmaxf(m_all, stats[(w * 16 + n) * 2]);
  float l_all = 0.f;
  float my_f = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = stats[(w * 16 + n) * 2];
    const float f = (mw == kNegInf) ? 0.f : fast_exp2(mw - m_all);
    l_all += stats[(w * 16 + n) * 2 + 1] * f;
    if (w == wave) my_f = f;
  }
  const bool empty = !(l_all > 0.f);
  const float sc = empty ? 0.f : (it.slot < 0 ? a.out_scale : 1.f) * my_f / l_all;
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) {
    const int dim = 16 * cb + 4 * g4;
    *(LDS_AS f32x4*)(mbuf + (wave * 16 + n) * kMergeRowFloats + dim) = st.o[cb] * sc;
  }
  __syncthreads();
  // wave w finalises dims [128w, 128w+128): lane -> row lane/4, 32 dims
  {
    const int row = lane >> 2;
    const int d0 = 128 * wave + 32 * (lane & 3);
    const RowInfo rj = row_info(a, it, row);
    if (rj.ok) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        f32x4 acc = {};
#pragma unroll
        for (int w = 0; w < 4; ++w) acc += *(LDS_AS f32x4*)(mbuf + (w * 16 + row) * kMergeRowFloats + d0 + 4 * q);
        store4(a, it, rj, row, d0 + 4 * q, acc);
      }
    }
  }
  if (wave == 0 && g4 == 0 && ri.ok) store_lse(a, it, ri, n, empty ? kNegInf : (m_all + __log2f(l_all)) * kLn2);
  __syncthreads();  // merge buffer overlaps stage 0 of the next item
}

// ---------------------------------------------------------------------------
// QUAD mode: a workgroup owns 32 rows.  Up to four sibling workgroups (same
// XCD, identical key ranges) hold the four 32-row slices of a row group, so
// the key stream is fetched once and re-served from L2.  Inside a workgroup
// the four waves split each 64-key stage for S = Q.K^T (wave w: keys
// [16w, 16w+16), all 32 rows) and split the 512 output columns for P.V
// (wave w: dims [128w, 128w+128), all 32 rows, all 64 keys); P goes through
// LDS.  All MFMAs are mfma_f32_16x16x32_bf16.
//
// The row max is shared: every wave computes P against the same running
// reference m, raised only when some wave's tile max passes m + kQuadSlack
// (log2 units).  Until then P <= 2^kQuadSlack, far inside bf16/fp32 range,
// and the exact softmax is unchanged.  The check reads all waves' tile
// maxima after the barrier that publishes P, so every wave takes the same
// branch; the raise path rescales O and l, recomputes P and re-publishes.
// ---------------------------------------------------------------------------
constexpr int kQuadRows = 32;
constexpr int kPRowBytes = 64 * 2 + 16;                       // P row: 64 keys bf16 + pad
constexpr int kPBufOff = 2 * kStageBytes;                      // after the two stages
constexpr int kTmaxOff = kPBufOff + kQuadRows * kPRowBytes;    // [4 waves][32 rows] float
constexpr int kQuadLdsBytes = kTmaxOff + 4 * kQuadRows * 4;
static_assert(kQuadLdsBytes <= 160 * 1024, "quad-mode LDS budget");
constexpr float kQuadSlack = 64.0f;

struct QuadState {
  f32x4 o[8][2];  // O^T tiles [col tile][row tile]: lane holds row 16t+n, dims 128w+16c+4g4+r
  float m[2];     // running reference max of rows n and 16+n (log2 units)
  float l[2];     // sum of P over this lane's keys, rows n and 16+n
};

__device__ __forceinline__ float max_xor16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

// P for this lane's 2 x 4 (row, key) values against reference m; writes them
// (bf16) to the P buffer and returns the fp32 values.
__device__ __forceinline__ void quad_write_p(LDS_AS char* __restrict__ pbuf, const float (&sv)[2][4],
                                             const float (&m)[2], float (&p)[2][4], int wave, int lane) {
  const int g4 = lane >> 4, n = lane & 15;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float mref = (m[t] == kNegInf) ? 0.f : m[t];
    i16x4 h;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[t][r] = fast_exp2(sv[t][r] - mref);
      h[r] = __builtin_bit_cast(short, (__bf16)p[t][r]);
    }
    *(LDS_AS i16x4*)(pbuf + (16 * t + n) * kPRowBytes + (16 * wave + 4 * g4) * 2) = h;
  }
}

template <int kPC>
__device__ __forceinline__ void quad_body(const AttnArgs& a, const bf16x8 (&qf)[2][18], QuadState& st,
                                          const LDS_AS char* __restrict__ cur, LDS_AS char* __restrict__ nxt,
                                          LDS_AS char* __restrict__ scr, bool prefetch, int page_base,
                                          int next_tok, int tok_end, int stage_tok, const int (&bound)[2],
                                          const int (&kb)[4], const int (&pb)[2], const int (&vb)[2],
                                          const int (&vx)[2], int wave, int lane, int page_hint) {
  // next stage's slices ride along Q.K^T; past the last stage they are
  // issued with an empty EXEC mask (addresses inside the request)
  StageLoader<kPC> ld;
  ld.begin(a, nxt, page_base, prefetch ? next_tok : stage_tok, tok_end, wave, page_hint);
  ld.on = __builtin_amdgcn_readfirstlane(prefetch ? ~0u : 0u);
  const int g4 = lane >> 4, n = lane & 15;
  LDS_AS char* pbuf = scr;
  LDS_AS float* tmax = (LDS_AS float*)(scr + (kTmaxOff - kPBufOff));

  // S^T tiles [16 keys x 16 rows] for row tiles 0 and 1; the K fragment is shared
  f32x4 sacc[2] = {f32x4{}, f32x4{}};
  auto kread = [&](int ks) -> bf16x8 {
    return ks < 16 ? lds_read_b128(cur, kb[ks & 3] + 256 * (ks >> 2)) : lds_read_b128(cur, pb[ks - 16]);
  };
  constexpr int KD = 4;  // K fragments in flight
  bf16x8 kr[KD];
#pragma unroll
  for (int i = 0; i < KD; ++i) kr[i] = kread(i);
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) {
    pin_loads();
    ld.issue(a, ks, wave);  // one prefetch slice per k-step
    const bf16x8 k0 = kr[ks % KD];
    if (ks + KD < 18) kr[ks % KD] = kread(ks + KD);
    sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[0][ks], sacc[0], 0, 0, 0);
    sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[1][ks], sacc[1], 0, 0, 0);
  }
  pin_loads();
  // scale, mask, tile max over this wave's 16 keys
  float sv[2][4], tm[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    tm[t] = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = stage_tok + 16 * wave + 4 * g4 + r;
      const float x = sacc[t][r] * a.scale_log2;
      sv[t][r] = tok < bound[t] ? x : kNegInf;
      tm[t] = fmaxf(tm[t], sv[t][r]);
    }
    tm[t] = max_xor16_32(tm[t]);
  }
  float p[2][4];
  quad_write_p(pbuf, sv, st.m, p, wave, lane);
  if (g4 == 0) {
    tmax[wave * kQuadRows + n] = tm[0];
    tmax[wave * kQuadRows + 16 + n] = tm[1];
  }
  __syncthreads();  // P and the tile maxima of all waves are published
  float smax[2];
  bool need = false;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    smax[t] = fmaxf(fmaxf(tmax[16 * t + n], tmax[kQuadRows + 16 * t + n]),
                    fmaxf(tmax[2 * kQuadRows + 16 * t + n], tmax[3 * kQuadRows + 16 * t + n]));
    need |= smax[t] > st.m[t] + kQuadSlack;
  }
  if (__builtin_amdgcn_ballot_w64(need) != 0) {  // same decision in every wave
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float m_new = fmaxf(st.m[t], smax[t]);
      const float alpha = (st.m[t] == kNegInf) ? 0.f : fast_exp2(st.m[t] - m_new);
      st.l[t] *= alpha;
      if (__builtin_amdgcn_ballot_w64(st.m[t] != kNegInf) != 0) {  // else O is still zero
#pragma unroll
        for (int c = 0; c < 8; ++c) scale_acc<4>(st.o[c][t], alpha);
      }
      st.m[t] = m_new;
    }
    // nobody has read P yet (only the tile maxima): rewrite it, publish again
    quad_write_p(pbuf, sv, st.m, p, wave, lane);
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) st.l[t] += (p[t][0] + p[t][1]) + (p[t][2] + p[t][3]);

  // O^T[128 dims x 32 rows] += V^T[128 dims x 64 keys] . P^T[64 keys x 32 rows]
  auto vread = [&](int j) -> bf16x8 {  // j = 8 kk + c: keys 32kk + 8g4 + 0..3, +4..7 of dims 128w + 16c + lane%16
    const int kk = j >> 3, c = j & 7;
    const int cx0 = (32 * c) ^ vx[0];
    const int cx1 = (32 * c) ^ vx[1];
    const i16x4 v0 = lds_read_tr(cur, vb[0] + cx0 + 32 * kk * kCkvRowBytes);
    const i16x4 v1 = lds_read_tr(cur, vb[1] + cx1 + 32 * kk * kCkvRowBytes);
    const i16x8 v = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    return __builtin_bit_cast(bf16x8, v);
  };
  constexpr int VD = 4;  // V^T fragments in flight
  bf16x8 vr[VD];
  bf16x8 pt[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int t = 0; t < 2; ++t) pt[kk][t] = lds_read_b128(pbuf, (16 * t + n) * kPRowBytes + (32 * kk + 8 * g4) * 2);
#pragma unroll
  for (int i = 0; i < VD; ++i) vr[i] = vread(i);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    pin_loads();
    const int kk = j >> 3, c = j & 7;
    const bf16x8 vf = vr[j % VD];
    if (j + VD < 16) vr[j % VD] = vread(j + VD);
    st.o[c][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pt[kk][0], st.o[c][0], 0, 0, 0);
    st.o[c][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pt[kk][1], st.o[c][1], 0, 0, 0);
  }
  pin_loads();
}

template <int kPC, bool kFp8>
__device__ void quad_item(const AttnArgs& a, const WorkItem& it, int role, LDS_AS char* smem, int wave,
                          int lane) {
  const int g4 = lane >> 4, n = lane & 15;
  const int rbase = kQuadRows * role;  // this workgroup's rows within the item's row group
  RowInfo ri[2];
  int bound[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    ri[t] = row_info(a, it, rbase + 16 * t + n);
    bound[t] = row_key_bound(a, it, ri[t]);
  }
  bf16x8 qf[2][18];
  {
    const bf16x8 z = {};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const __bf16* qn = (const __bf16*)a.q_nope + ri[t].qrow * a.q_stride + 8 * g4;
      const __bf16* qp = (const __bf16*)a.q_pe + ri[t].qrow * a.qpe_stride + 8 * g4;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qf[t][ks] = ri[t].ok ? *(const bf16x8*)(qn + 32 * ks) : z;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) qf[t][16 + ks] = ri[t].ok ? *(const bf16x8*)(qp + 32 * ks) : z;
    }
  }
  // LDS base offsets: K reads (as in the narrow mode), V^T reads
  int kb[4], pb[2], vb[2], vx[2];
  {
    const int t = wave * 16 + n;
#pragma unroll
    for (int k = 0; k < 4; ++k) kb[k] = ckv_off(t, 4 * k + g4);
#pragma unroll
    for (int k = 0; k < 2; ++k) pb[k] = kpe_off(t, 4 * k + g4);
    const int q = (lane & 15) >> 2;
    const int x = (lane & 3) >> 1;
    const int w8 = (lane & 1) ? 8 : 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * g4 + q + 4 * h;    // key row within a 32-key half (mod 16 fixes the swizzle)
      const int sw = ckv_swz(row);
      vb[h] = row * kCkvRowBytes + 256 * wave + ((x ^ (sw & 1)) << 4) + w8;
      vx[h] = (sw & 14) << 4;                 // chunk 2c of column tile c lands at (2c ^ (sw & 14))
    }
  }

  QuadState st;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    st.o[c][0] = f32x4{};
    st.o[c][1] = f32x4{};
  }
  st.m[0] = st.m[1] = kNegInf;
  st.l[0] = st.l[1] = 0.f;

  LDS_AS char* scr = smem + kPBufOff;
  const int page_base = ld_const(a.kv_indptr, it.b);
  const int nstage = (it.tok1 - it.tok0 + kStageTokens - 1) / kStageTokens;
  if (nstage > 0) issue_stage_bf16<kPC>(a, smem, page_base, it.tok0, it.tok1, wave, lane);
  // one-page stages: the page of stage s+1 is looked up a stage ahead (stage 0's when none is next)
  auto page_at = [&](int stage) -> int {
    return kPC == kPageBig ? ld_const(a.kv_indices, page_base + ((it.tok0 + stage * kStageTokens) >> a.page_shift))
                           : -1;
  };
  int pg_next = page_at(nstage > 1 ? 1 : 0);
  for (int s = 0; s < nstage; ++s) {
    const int pg_after = page_at(s + 2 < nstage ? s + 2 : 0);
    wait_vmcnt<0>();
    __syncthreads();  // stage s landed; every wave is done with stage s-1
    quad_body<kPC>(a, qf, st, smem + (s & 1) * kStageBytes, smem + ((s + 1) & 1) * kStageBytes, scr,
                   s + 1 < nstage, page_base, it.tok0 + (s + 1 < nstage ? s + 1 : 0) * kStageTokens, it.tok1,
                   it.tok0 + s * kStageTokens, bound, kb, pb, vb, vx, wave, lane, pg_next);
    pg_next = pg_after;
  }

  // row sums: this lane's keys -> this wave's keys -> all waves
  LDS_AS float* lsum = (LDS_AS float*)(smem + kTmaxOff);
  float lw[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    lw[t] = st.l[t] + __shfl_xor(st.l[t], 16);
    lw[t] += __shfl_xor(lw[t], 32);
  }
  __syncthreads();  // the last stage's tile maxima have been read
  if (g4 == 0) {
    lsum[wave * kQuadRows + n] = lw[0];
    lsum[wave * kQuadRows + 16 + n] = lw[1];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = 16 * t + n;
    const float L = (lsum[r] + lsum[kQuadRows + r]) + (lsum[2 * kQuadRows + r] + lsum[3 * kQuadRows + r]);
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : (it.slot < 0 ? a.out_scale : 1.f) / L;
    if (ri[t].ok) {
#pragma unroll
      for (int c = 0; c < 8; ++c) store4(a, it, ri[t], rbase + r, 128 * wave + 16 * c + 4 * g4, st.o[c][t] * inv);
      if (wave == 0 && g4 == 0) store_lse(a, it, ri[t], rbase + r, empty ? kNegInf : (st.m[t] + __log2f(L)) * kLn2);
    }
  }
  __syncthreads();  // LDS is reused by the next item
}

template <int kPC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_attn_quad_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kQuadLdsBytes];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // workgroup -> (virtual unit, role); siblings of a unit share blockIdx.x mod 8 (one XCD)
  const int G = a.group_size;
  int vcu, role;
  if (a.xcd_map) {
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
    vcu = x + 8 * (slot / G);
    role = slot - (slot / G) * G;
  } else {
    vcu = blockIdx.x / G;
    role = blockIdx.x - vcu * G;
  }
  if (vcu >= a.num_wgs) return;
  const int i0 = ld_const(a.wg_ptr, vcu);
  const int i1 = ld_const(a.wg_ptr, vcu + 1);
  for (int i = i0; i < i1; ++i) {
    const int32_t* ip = (const int32_t*)(a.items + i);
    WorkItem it;
    it.b = ld_const(ip, 0);
    it.row0 = ld_const(ip, 1);
    it.nrows = ld_const(ip, 2);
    it.tok0 = ld_const(ip, 3);
    it.tok1 = ld_const(ip, 4);
    it.kv_len = ld_const(ip, 5);
    it.q_len = ld_const(ip, 6);
    it.slot = ld_const(ip, 7);
    if (!clip_live(a, it)) continue;
    if (kQuadRows * role >= it.nrows) continue;  // this slice of the row group is empty
    quad_item<kPC, false>(a, it, role, smem, wave, lane);
  }
}

// ---------------------------------------------------------------------------
// Combine: merge the partial results of each split (request, row block).
// out = sum_s w_s o_s / sum_s w_s with w_s = exp(lse_s - max lse), and
// lse = max lse + ln sum w (the log-sum-exp identity).  One wave per row:
// lane l owns dims 8l..8l+7.  The split lse values (and partial maxima) are
// wave-uniform, so they are scalar loads that every lane uses directly: the
// maximum and the weights need no cross-lane step.  The partial rows of the
// first 8 splits are loaded together with them, so a row with at most 8
// splits costs one memory round trip.
// ---------------------------------------------------------------------------
constexpr int kCombineRows = 4;  // rows per combine workgroup (one per wave)
constexpr int kCombineBatch = 8;  // partial rows in flight per lane

__device__ __forceinline__ float ld_const_f(const float* p, size_t i) {
  return __builtin_bit_cast(float, ((const CONST_AS int32_t*)p)[i]);
}

__device__ __forceinline__ void combine_row(const AttnArgs& a, int gi, int r, int lane) {
  const int32_t* gp = (const int32_t*)(a.groups + gi);
  const int g_b = ld_const(gp, 0), g_row0 = ld_const(gp, 1), g_nrows = ld_const(gp, 2);
  const int nsplit = ld_const(gp, 3), slot0 = ld_const(gp, 4);
  if (r >= g_nrows) return;
  if (a.live_kv_len != nullptr && a.live_q) {
    // capacity prefill: rows past the request's live query tokens were not computed
    const int n = min(max(ld_const(a.qo_indptr, g_b + 1) - ld_const(a.qo_indptr, g_b), 0), ld_const(gp, 5));
    if (g_row0 + r >= n * a.num_heads) return;
  }
  const int q_start = a.qo_indptr ? ld_const(a.qo_indptr, g_b) : g_b;
  const size_t row0 = (size_t)slot0 * a.rows_per_block + r;  // row r of the group's first slot
  const size_t stride = (size_t)a.rows_per_block;             // rows between consecutive slots
  const int d0 = lane * 8;
  auto prow = [&](int sp) { return *(const bf16x8*)(a.part_o + (row0 + (size_t)sp * stride) * kDimCkv + d0); };
  auto lse_at = [&](int sp) { return ld_const_f(a.part_lse, row0 + (size_t)sp * stride); };
  bf16x8 v[kCombineBatch];
  float ls[kCombineBatch];
#pragma unroll
  for (int j = 0; j < kCombineBatch; ++j) {
    if (j < nsplit) {
      v[j] = prow(j);
      ls[j] = lse_at(j);
    } else {
      ls[j] = kNegInf;
    }
  }
  float M = kNegInf;
#pragma unroll
  for (int j = 0; j < kCombineBatch; ++j) M = fmaxf(M, ls[j]);
  for (int sp = kCombineBatch; sp < nsplit; ++sp) M = fmaxf(M, lse_at(sp));
  float W = 0.f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (M != kNegInf) {
    for (int c = 0; c < nsplit; c += kCombineBatch) {
      if (c > 0) {
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) {
          if (c + j < nsplit) {
            v[j] = prow(c + j);
            ls[j] = lse_at(c + j);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j) {
        if (c + j < nsplit) {
          const float w = (ls[j] == kNegInf) ? 0.f : __expf(ls[j] - M);
          W += w;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += w * (float)v[j][e];
        }
      }
    }
  }
  const int H = a.num_heads;
  const int rr = g_row0 + r;
  const int qi = rr / H;
  const size_t qrow = (size_t)(q_start + qi) * H + (rr - qi * H);
  float den = W;
  if (a.attn_sink != nullptr && W > 0.f) den += __expf(a.attn_sink[rr - qi * H] - M);  // the sink's share
  const float inv = (W > 0.f) ? a.out_scale / den : 0.f;
  if (a.max_logits != nullptr && lane == 0) {
    float mx = kNegInf;
    for (int sp = 0; sp < nsplit; ++sp) mx = fmaxf(mx, ld_const_f(a.part_max, row0 + (size_t)sp * stride));
    a.max_logits[qrow] = mx;
  }
  if (a.out_bf16) {
    bf16x8 h;
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = (__bf16)(acc[j] * inv);
    *(bf16x8*)((__bf16*)a.out + qrow * kDimCkv + d0) = h;
  } else {
    f32x4* dst = (f32x4*)((float*)a.out + qrow * kDimCkv + d0);
    dst[0] = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    dst[1] = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  }
  if (lane == 0) a.lse[lse_index(a, g_b, rr, qrow)] = (W > 0.f) ? M + __logf(W) : kNegInf;
}

__global__ __launch_bounds__(256) void mla_combine_kernel(AttnArgs a) {
  const int chunks_per_group = a.rows_per_block / kCombineRows;
  const int gi = blockIdx.x / chunks_per_group;
  const int r = (blockIdx.x - gi * chunks_per_group) * kCombineRows + (threadIdx.x >> 6);
  combine_row(a, gi, r, threadIdx.x & 63);
}


// Workgroup -> work list.  Workgroups are dealt to the 8 XCDs round-robin
// (blockIdx mod 8); lists are numbered so that consecutive lists land on
// one XCD.  The planner fills lists in request order, so the pieces of a
// split request, or the row blocks of a prefill request, share an L2 (their
// query rows, and keys read at the same time, come from HBM once).  A
// bijection for any list count n: XCD x runs ceil((n - x) / 8) lists.
__device__ __forceinline__ int xcd_list(int b, int n) {
  const int x = b & 7;
  int base = 0;
#pragma unroll
  for (int y = 0; y < 7; ++y) base += (y < x) ? (n - y + 7) >> 3 : 0;
  return base + (b >> 3);
}

template <int kMode, int kPC, bool kFp8, bool kSparse = false, bool kQ8 = false, bool kM1 = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char
      smem_raw[kFp8 ? kFp8LdsBytes : (kMode == 1 && !kSparse ? kDsLdsBytes : kLdsBytes)];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int list = xcd_list(blockIdx.x, a.num_wgs);
  const int i0 = ld_const(a.wg_ptr, list);
  const int i1 = ld_const(a.wg_ptr, list + 1);
  for (int i = i0; i < i1; ++i) {
    const int32_t* ip = (const int32_t*)(a.items + i);
    WorkItem it;
    it.b = ld_const(ip, 0);
    it.row0 = ld_const(ip, 1);
    it.nrows = ld_const(ip, 2);
    it.tok0 = ld_const(ip, 3);
    it.tok1 = ld_const(ip, 4);
    it.kv_len = ld_const(ip, 5);
    it.q_len = ld_const(ip, 6);
    it.slot = ld_const(ip, 7);
    if (kSparse) {
      // the list's valid keys were counted on the device: pieces past them are empty
      const int L = ld_const(a.sparse_len, it.b);
      it.kv_len = L;
      it.tok1 = max(it.tok0, min(it.tok1, L));
    } else if (!clip_live(a, it)) {
      continue;
    }
    if (kMode == 1 && kFp8) {
      wide8_item<kPC, kSparse, kQ8, typename std::conditional<kM1, FmtM1, FmtV32>::type>(a, it, smem, wave, lane);
    } else if (kMode == 1 && !kSparse) {
      ds_item<kPC>(a, it, smem, wave);
    } else if (kMode == 1) {
      wide_item<kPC, kSparse>(a, it, smem, wave, lane);
    } else {
      narrow_item<kPC, kFp8, kM1>(a, it, smem, wave, lane);
    }
  }
}


}  // namespace

// Attention launches go through hipExtLaunchKernelGGL so that optional
// timing events are recorded by the kernel's own dispatch (start and end of
// its execution, no queue gaps); with null events it is a plain launch.
template <int kMode, int kPC>
hipError_t launch_mode(const AttnArgs& a, int kv_fp8, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (kv_fp8 == 2) {
    hipExtLaunchKernelGGL((mla_attn_kernel<kMode, kPC, true, false, false, true>), dim3(a.num_wgs), dim3(256), 0,
                          stream, t0, t1, 0, a);
  } else if (kv_fp8) {
    hipExtLaunchKernelGGL((mla_attn_kernel<kMode, kPC, true>), dim3(a.num_wgs), dim3(256), 0, stream, t0, t1, 0, a);
  } else {
    hipExtLaunchKernelGGL((mla_attn_kernel<kMode, kPC, false>), dim3(a.num_wgs), dim3(256), 0, stream, t0, t1, 0, a);
  }
  return hipGetLastError();
}

template <int kPC>
hipError_t launch_quad(const AttnArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  hipExtLaunchKernelGGL((mla_attn_quad_kernel<kPC>), dim3(a.grid), dim3(256), 0, stream, t0, t1, 0, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int tile_mode, int kv_fp8, hipStream_t stream, hipEvent_t t0,
                            hipEvent_t t1) {
  if (a.num_wgs <= 0) return hipSuccess;
  const int pc = a.page_shift >= 6 ? kPageBig : (a.page_shift >= 3 ? kPageMid : kPageSmall);
  if (tile_mode == 3) {
    if (kv_fp8) return hipErrorNotSupported;  // rejected when the plan is made
    if (pc == kPageBig) return launch_quad<kPageBig>(a, stream, t0, t1);
    if (pc == kPageMid) return launch_quad<kPageMid>(a, stream, t0, t1);
    return launch_quad<kPageSmall>(a, stream, t0, t1);
  }
  if (tile_mode == 1) {
    if (pc == kPageBig) return launch_mode<1, kPageBig>(a, kv_fp8, stream, t0, t1);
    if (pc == kPageMid) return launch_mode<1, kPageMid>(a, kv_fp8, stream, t0, t1);
    return launch_mode<1, kPageSmall>(a, kv_fp8, stream, t0, t1);
  }
  if (pc == kPageBig) return launch_mode<2, kPageBig>(a, kv_fp8, stream, t0, t1);
  if (pc == kPageMid) return launch_mode<2, kPageMid>(a, kv_fp8, stream, t0, t1);
  return launch_mode<2, kPageSmall>(a, kv_fp8, stream, t0, t1);
}

hipError_t launch_attention_q8(const AttnArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (a.num_wgs <= 0) return hipSuccess;
  const int pc = a.page_shift >= 6 ? kPageBig : (a.page_shift >= 3 ? kPageMid : kPageSmall);
  if (pc == kPageBig) {
    hipExtLaunchKernelGGL((mla_attn_kernel<1, kPageBig, true, false, true>), dim3(a.num_wgs), dim3(256), 0, stream,
                          t0, t1, 0, a);
  } else if (pc == kPageMid) {
    hipExtLaunchKernelGGL((mla_attn_kernel<1, kPageMid, true, false, true>), dim3(a.num_wgs), dim3(256), 0, stream,
                          t0, t1, 0, a);
  } else {
    hipExtLaunchKernelGGL((mla_attn_kernel<1, kPageSmall, true, false, true>), dim3(a.num_wgs), dim3(256), 0, stream,
                          t0, t1, 0, a);
  }
  return hipGetLastError();
}

hipError_t launch_sparse_attention(const AttnArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1, bool m1) {
  if (a.num_wgs <= 0) return hipSuccess;
  if (a.page_shift != 0 || a.sparse_len == nullptr) return hipErrorInvalidValue;
  if (a.kv_fp8 != nullptr && m1) {
    hipExtLaunchKernelGGL((mla_attn_kernel<1, kPageSmall, true, true, false, true>), dim3(a.num_wgs), dim3(256), 0,
                          stream, t0, t1, 0, a);
  } else if (a.kv_fp8 != nullptr) {
    hipExtLaunchKernelGGL((mla_attn_kernel<1, kPageSmall, true, true>), dim3(a.num_wgs), dim3(256), 0, stream, t0,
                          t1, 0, a);
  } else {
    hipExtLaunchKernelGGL((mla_attn_kernel<1, kPageSmall, false, true>), dim3(a.num_wgs), dim3(256), 0, stream, t0,
                          t1, 0, a);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const AttnArgs& a, hipStream_t stream) {
  if (a.num_groups <= 0) return hipSuccess;
  const int chunks = a.rows_per_block / kCombineRows;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(a.num_groups * chunks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
