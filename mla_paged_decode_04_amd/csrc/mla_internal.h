// Internal declarations shared by the translation units of the paged MLA
// decode library: problem constants, the split-plan arithmetic used by both
// the host and the device planner, device helpers (fp8 -> bf16, LDS DMA,
// transposed LDS reads) and the parameter block of the decode kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "mla_decode.h"

namespace mla_detail {
constexpr int D = MLA_D_QK;          // 576
constexpr int DV = MLA_D_V;          // 512
constexpr int NT = 64;               // key granularity of split chunks
constexpr int NTHREADS = 256;        // 4 wave64 per workgroup
constexpr int OSTRIDE = DV + 4;      // fp32 row stride of the output staging
constexpr int ITEM_INTS = 8;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
// Online softmax with a lazily moved reference max (base 2): probabilities
// are exp2(score - m_ref) with m_ref the row max of the first tile that row
// saw. Later scores up to m_ref + BIG_SLACK are accumulated as they are
// (p <= 2^64 is exact enough in bf16 and fp32: relative precision does not
// depend on magnitude), so the accumulators are never rescaled in the fast
// loop. A larger jump switches the work item to a slow loop that rescales.
constexpr float BIG_SLACK = 64.0f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef short s16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

// Two OCP e4m3fn codes (bytes 0,1 of `w`, or bytes 2,3 when `hi`) to two
// bf16 packed in one dword, by gfx950's v_cvt_scalef32_pk_bf16_fp8 with scale
// 1. Every e4m3fn value is a bf16 value, so the conversion is exact.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  bf16x2_t r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, true)
                  : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  uint4 r;
  r.x = fp8x2_to_bf16x2(w0, false);
  r.y = fp8x2_to_bf16x2(w0, true);
  r.z = fp8x2_to_bf16x2(w1, false);
  r.w = fp8x2_to_bf16x2(w1, true);
  return r;
}

// Four float32 values x (|x| < 256) -> e4m3fn codes of hi = nearest(x) and
// lo = nearest(x - hi), packed four to a dword. For x = q * 2^e with q a bf16
// value (8 significant bits) the residual x - hi is a multiple of q's last
// place with at most 4 significant bits, so lo is exact and hi + lo = x
// whenever that place is at least e4m3fn's smallest step 2^-9 (elements down
// to 2^-10 of a row maximum scaled to [128, 256); smaller ones lose bits
// below 2^-18 of the row maximum).
__device__ __forceinline__ void split_fp8x4(float x0, float x1, float x2, float x3, uint32_t& hi,
                                            uint32_t& lo) {
  s16x2_t h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2_t{0, 0}, x0, x1, 1.0f, false);
  h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, x2, x3, 1.0f, true);
  hi = __builtin_bit_cast(uint32_t, h);
  const uint32_t d01 = fp8x2_to_bf16x2(hi, false), d23 = fp8x2_to_bf16x2(hi, true);   // exact
  const float r0 = x0 - __builtin_bit_cast(float, d01 << 16);
  const float r1 = x1 - __builtin_bit_cast(float, d01 & 0xFFFF0000u);
  const float r2 = x2 - __builtin_bit_cast(float, d23 << 16);
  const float r3 = x3 - __builtin_bit_cast(float, d23 & 0xFFFF0000u);
  s16x2_t l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2_t{0, 0}, r0, r1, 1.0f, false);
  l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, r2, r3, 1.0f, true);
  lo = __builtin_bit_cast(uint32_t, l);
}

// 8 bf16 (one uint4) times 2^e -> hi and lo codes, two dwords each.
__device__ __forceinline__ void split_fp8x8(uint4 v, float mul, uint32_t* hi, uint32_t* lo) {
  auto f = [](uint32_t w, bool upper) {
    return __builtin_bit_cast(float, upper ? (w & 0xFFFF0000u) : (w << 16));
  };
  split_fp8x4(f(v.x, false) * mul, f(v.x, true) * mul, f(v.y, false) * mul, f(v.y, true) * mul, hi[0], lo[0]);
  split_fp8x4(f(v.z, false) * mul, f(v.z, true) * mul, f(v.w, false) * mul, f(v.w, true) * mul, hi[1], lo[1]);
}

__device__ __forceinline__ float wave_max_across_groups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float wave_sum_across_groups(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  // one v_cvt_pk_bf16_f32 (round to nearest even)
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// Transposed 64-bit LDS read (see the V^T operand set-up in the decode kernel).
__device__ __forceinline__ s16x4_t read_vt(const char* p) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
  // generic -> LDS address space needs a C-style cast
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
}

// One wave-wide 1 KB transfer HBM -> LDS: lane l's 16 bytes at gbase + voff
// land at LDS byte address lds + 16*l (global_load_lds_dwordx4, saddr form).
// Issued from inline asm: the compiler neither sees nor waits on it, so all
// ordering against LDS reads is done with the explicit vmcnt waits below.
// (M0 carries the LDS address; nothing else in these kernels uses M0.)
// Pin a wave-uniform value into SGPRs (the "s" asm constraints below need it).
__device__ __forceinline__ const char* uniform_ptr(const char* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ void lds_dma16(const char* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform_ptr(gbase))
               : "memory");
}

// Same with the non-temporal hint: data that is read exactly once streams
// through the caches (measured on MI355X: 6.9 TB/s vs 5.8 TB/s for a plain
// HBM -> LDS copy of 1.2 GB).
__device__ __forceinline__ void lds_dma16_nt(const char* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform_ptr(gbase))
               : "memory");
}

// 16 bytes at p (always a valid address) if keep, else zeros: the load is
// issued unconditionally and masked. A branch around a load leaves the
// compiler without an exact count of the memory operations in flight, and
// its next wait then drains all of them, the DMAs it cannot see included.
__device__ __forceinline__ uint4 load16_masked(const void* p, bool keep) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t m = keep ? 0xFFFFFFFFu : 0u;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// Store layout for four MFMA result fragments of a 16-row tile, packed to
// 16-bit values: pk[i][0..1] of lane (c16, g) hold columns 16 i + 4 g .. + 3
// of row c16. Rearranged across lanes so that two 16-byte stores per lane
// write 8 whole rows of the tile's 64 columns each (128 bytes, one cache
// line per row): `lo` for rows 0..7, `hi` for rows 8..15, lane (c16, g)
// writing row (c16 & 7) (+ 8) at byte whole_row_col(c16, g) of the row's
// slice. Two v_permlane16_swap per fragment pair turn the 4-column pieces
// of lanes g and g + 1 into 8-column runs (columns {0, 16, 8, 24}[g] and
// + 32 of the 64); a DPP row rotate by 8 then swaps the second run of rows
// 0..7 with the first run of rows 8..15. Every lane of the wave must take
// part. (Half- or quarter-line stores keep fewer writes in flight.)
__device__ __forceinline__ void whole_row_runs(uint32_t (&pk)[4][2], int c16, uint4& lo, uint4& hi) {
#pragma unroll
  for (int pr = 0; pr < 4; pr += 2)
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const auto sw = __builtin_amdgcn_permlane16_swap(pk[pr][d], pk[pr + 1][d], false, false);
      pk[pr][d] = sw[0];
      pk[pr + 1][d] = sw[1];
    }
  const uint4 ra = make_uint4(pk[0][0], pk[0][1], pk[1][0], pk[1][1]);
  const uint4 rb = make_uint4(pk[2][0], pk[2][1], pk[3][0], pk[3][1]);
  const bool low = c16 < 8;
  const uint4 x = low ? rb : ra;
  constexpr int ROW_ROR8 = 0x128;   // DPP row_ror:8: lane l of a 16-lane row reads lane l ^ 8
  const uint4 y = make_uint4(static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x.x), ROW_ROR8, 0xF, 0xF, false)),
                             static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x.y), ROW_ROR8, 0xF, 0xF, false)),
                             static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x.z), ROW_ROR8, 0xF, 0xF, false)),
                             static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x.w), ROW_ROR8, 0xF, 0xF, false)));
  lo = low ? ra : y;
  hi = low ? y : rb;
}
__device__ __forceinline__ int whole_row_col(int c16, int g) {
  return 2 * ((g & 1) * 16 + (g >> 1) * 8) + (c16 < 8 ? 0 : 64);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}

// Compiler fence: keeps LDS reads/writes and DMA issue in program order around
// the explicit waits below (the compiler does not model DMA-written LDS).
__device__ __forceinline__ void mem_fence_compiler() { asm volatile("" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Split partials leave as fp16 values of o * 2^k, with a per-row k that puts
// the row's largest |o| in [2^14, 2^15): every element keeps 11 bits relative
// to the row maximum, nothing overflows, and the partial traffic (written by
// the decode kernels, read back by the combine) is half that of fp32.
__device__ __forceinline__ int partial_exponent(float amax) {
  return amax > 0.f && amax < INFINITY ? 15 - __builtin_amdgcn_frexp_expf(amax) : 0;
}

// Bits of the workspace header's flag word ([3]).
constexpr int FLAG_SEQ_LEN_CLAMPED = 1;   // a seq_len was outside [0, max_blocks * bs]
constexpr int FLAG_PLAN_OVERFLOW = 2;     // the plan did not fit the workspace bounds
constexpr int FLAG_BAD_PAGE = 4;          // a block-table entry in range was outside [0, num_blocks)
constexpr int FLAG_BAD_ITEM = 8;          // the workspace plan did not fit this call: items skipped

// Record (once per wave) that a tile's page id was outside [0, num_blocks):
// the tile was read from page 0, zeroed, and its keys masked out. Called after
// the last tile wait, so the atomic does not disturb the DMA vmcnt counting.
__device__ __forceinline__ void flag_bad_page(int32_t* flags, bool bad) {
  if (bad && (threadIdx.x & 63) == 0)
    __hip_atomic_fetch_or(flags, FLAG_BAD_PAGE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct FwdParams;
__device__ __forceinline__ void flag_bad_item(int32_t* flags) {
  if (threadIdx.x == 0)
    __hip_atomic_fetch_or(flags, FLAG_BAD_ITEM, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct FwdParams {
  const uint16_t* q;
  const uint8_t* kv;
  const int32_t* block_table;
  const int32_t* seq_lens;
  uint16_t* out;
  float* lse;
  const int32_t* header;
  int32_t* flags;     // header word 3: decode kernels OR in FLAG_BAD_PAGE
  const int32_t* items;
  _Float16* part_o;   // split partials: fp16 rows of o * 2^part_scale
  float* part_lse;     // base-2 lse per partial row
  int32_t* part_scale; // per partial row
  int heads, s_q, rows, bs, max_blocks, max_keys, causal, num_blocks;
  int batch, max_items, max_slots;   // bounds of the plan this call can run
  float scale_log2;   // softmax_scale * kv_scale * log2(e)
  float out_scale;    // kv_scale
};

// A work item is checked before any index is formed from it: the plan in the
// workspace comes from an earlier call when it is reused (mla_decode_with_plan,
// mla_decode_fwd_only), and a stale or foreign plan must not send the kernels
// outside their buffers. An item that fails is skipped and FLAG_BAD_ITEM set.
// (Items start on 64-key boundaries, which the tile addressing relies on.)
__device__ __forceinline__ bool item_in_range(const FwdParams& p, int rgs, int b, int rg, int t0, int t1,
                                              int slot) {
  return b >= 0 && b < p.batch && rg >= 0 && rg * rgs < p.rows && t0 >= 0 && (t0 & (NT - 1)) == 0 &&
         t0 <= t1 && t1 <= p.max_keys && slot < p.max_slots;
}

// Decode-kernel launchers (one per translation unit); the grid is one
// workgroup per potential work item.
void launch_narrow(int kv_dtype, dim3 grid, hipStream_t st, const FwdParams& fp);
void launch_wide(int kv_dtype, dim3 grid, hipStream_t st, const FwdParams& fp);
void launch_wide128(int kv_dtype, dim3 grid, hipStream_t st, const FwdParams& fp);

}  // namespace mla_detail
