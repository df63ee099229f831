// Paged MLA decode, > 64 query rows per sequence (the 128-head cases):
// decode attention of MLA in its MQA form ("[WIP][Attention] FlashAttn MLA",
// description) with 128 query rows per work item, 32 per wave, on gfx950's
// 32x32x16 bf16 MFMA. A 32-row MFMA tile feeds each LDS byte of K or V to 32
// rows (twice the 16-row tiles), and issues at full rate with one wave per
// SIMD. With fp8 e4m3fn caches ("[Attention] Blackwell FP8 MLA support with
// CUTLASS_MLA backend", Test Plan) the scores run on the 32x32x64 fp8 MFMA
// against an exact two-term fp8 split of q, and V is widened to bf16 in
// registers right before each PV MFMA.
#include <type_traits>

#include "mla_internal.h"

using namespace mla_detail;

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// The ring: 4 slots of 36864 bytes (32 bf16 keys or 64 fp8 keys of 576
// dims), three in flight while one is computed, one workgroup barrier per
// slot. Each wave issues 9 of the 36 wave-wide 1 KB transfers of a slot.
constexpr int X_TILE = 36864;
constexpr int X_SLOTS = 4;
constexpr int X_NDMA = 9;
constexpr int X_GSTRIDE = 4096;   // bytes per 64-dim column group (both layouts)
constexpr int X_RGS = 128;        // query rows per work item
constexpr int X_STEP = 32;        // keys per compute step (one 32x32 S block)
#ifndef QK_AHEAD
#define QK_AHEAD 4                // k-steps whose K reads are issued ahead
#endif
#ifndef PV_AHEAD
#define PV_AHEAD 8                // PV MFMAs whose V^T reads are issued ahead
#endif

// bf16 slot layout: [9 column groups][32 keys][8 x 16-byte chunks], chunk c of
// key k at position c ^ swz16(k). The swizzle is a bijection of key bits 1-3
// (for either parity of bit 0), so the 16-byte K reads of 16 consecutive keys
// hit 16 distinct bank groups; and it flips bit 2 between keys k and k + 2, so
// the transposed V reads (4 keys x 32 dims per 32 lanes) are conflict-free too.
__device__ __forceinline__ int swz16(int k) {
  return (((k >> 1) & 1) << 2) | (((k >> 3) & 1) << 1) | ((k >> 2) & 1);
}
// fp8 slot layout: [9 column groups][64 keys][4 x 16-byte chunks], chunk c of
// key k at position c ^ ((k >> 2) & 3).
__device__ __forceinline__ int swz8(int k) { return (k >> 2) & 3; }

// Lanes l and l ^ 32 hold the two halves of one row's 32 scores: combine them
// with gfx950's v_permlane32_swap (see the wide kernel for why inline asm).
__device__ __forceinline__ float halves_max(float v) {
  float y = v;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(v), "+v"(y));
  return fmaxf(v, y);
}
__device__ __forceinline__ float halves_sum(float v) {
  float y = v;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(v), "+v"(y));
  return v + y;
}

// The lane id, read afresh where it is used: an opaque asm the compiler can
// neither merge with other reads nor hoist out of the loop. Lane constants
// derived from it are recomputed at each use (a few VALU instructions that
// run under the MFMAs) rather than kept live across the tile loop, where the
// register pressure would send them to scratch, and the wait for a scratch
// reload would also wait for every tile transfer in flight.
__device__ __forceinline__ int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// The S^T accumulation chain is issued from inline asm so that S lives in
// VGPRs: through the builtin the compiler gives every MFMA accumulator an
// AGPR, and S (16) next to O (256) overflows the 256 AGPRs into spills. The
// asm carries the hazard waits the compiler would otherwise add: a chained
// MFMA reading exactly the previous one's result needs none; an operand
// written by a VALU instruction needs 2 wait states before the MFMA reads it
// (the _v forms); and VALU reads of the result wait for the last MFMA's
// passes (qk_done, which also orders those reads after it).
__device__ __forceinline__ void qk_first(f32x16_t& s, const bf16x8_t& a, const bf16x8_t& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_next(f32x16_t& s, const bf16x8_t& a, const bf16x8_t& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_first_v(f32x16_t& s, const bf16x8_t& a, const bf16x8_t& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_next_v(f32x16_t& s, const bf16x8_t& a, const bf16x8_t& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_done(f32x16_t& s) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
}

// fp8 caches: S^T on gfx950's 32x32x64 MFMA with both operands e4m3fn, the
// keys' codes as stored and q split per row into q * 2^e = hi + lo (below).
// Same chain rules as the bf16 forms; VALU reads of the result wait for the
// 16 passes of the last MFMA (qk8_done).
__device__ __forceinline__ void qk8_first(f32x16_t& s, const i32x8_t& a, const i32x8_t& b) {
  asm("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk8_next(f32x16_t& s, const i32x8_t& a, const i32x8_t& b) {
  asm("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk8_first_v(f32x16_t& s, const i32x8_t& a, const i32x8_t& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk8_next_v(f32x16_t& s, const i32x8_t& a, const i32x8_t& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk8_done(f32x16_t& s) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
}

// LDS reads by 32-bit LDS byte address. The per-lane operand offsets are
// formed as (slot base + lane offset) ^ (swizzle flip): the slot base is a
// multiple of 1024, so the XOR only touches the lane offset's chunk bits, and
// the result changes every step, which keeps the compiler from hoisting the
// flipped variants out of the loop as extra live registers.
__device__ __forceinline__ bf16x8_t lds_b128(uint32_t a) {
  return *(const __attribute__((address_space(3))) bf16x8_t*)(a);
}
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t lds_u128(uint32_t a) {
  return *(const __attribute__((address_space(3))) u32x4_t*)(a);
}
__device__ __forceinline__ s16x4_t lds_tr16(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(a));
}
__device__ __forceinline__ uint2 lds_tr8(uint32_t a) {
  return __builtin_bit_cast(
      uint2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(a)));
}

// MFMA operand layouts (32x32x16): A[m][k] and B[k][n] put m (or n) = lane & 31
// and k = 8 * (lane >> 5) + i in element i; C[m][n] puts n = lane & 31 and
// m = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3) in element e.
//   S^T (32 keys x 32 rows) = K (A, from LDS) . Q^T (B, registers)
//   O^T (512 dims x 32 rows) += V^T (A, transposed LDS reads) . P^T (B)
// The C layout of S^T gives lane (row n, half h) the keys 8q + 4h + r; packed
// in that order they are exactly the P^T operand of the two 16-key PV steps
// once the V^T operand of step s takes keys 16s + 4h + (0..3) and
// 16s + 8 + 4h + (0..3), which two 4-key transposed reads deliver.
template <int KVT>
__global__ __launch_bounds__(NTHREADS, 1) void mla_decode_wide128(FwdParams p) {
  constexpr bool F8 = KVT == MLA_DTYPE_FP8_E4M3FN;
  constexpr int KT = F8 ? 64 : 32;                  // keys per ring slot
  constexpr int ROWB = F8 ? D : D * 2;              // bytes per cached row
  __shared__ __attribute__((aligned(1024))) char smem[X_SLOTS * X_TILE];   // 147456 bytes
  // the rope part of Q (the last 4 k-steps), 128 rows x 128 bytes: in LDS
  // rather than in registers, which keeps the fast loop free of spills
  __shared__ __attribute__((aligned(1024))) char qrope[X_RGS * 128];        // 16384 bytes

  // XCD-aware item order (consecutive workgroups go to different XCDs): each
  // XCD takes a contiguous run of items. The grid is a multiple of 8.
  const int n_items = min(p.header[0], p.max_items);
  const int per_xcd = (n_items + 7) >> 3;
  const int xw = blockIdx.x;
  if ((xw >> 3) >= per_xcd) return;
  const int item_id = (xw & 7) * per_xcd + (xw >> 3);
  if (item_id >= n_items) return;
  const int32_t* it = p.items + (size_t)item_id * ITEM_INTS;
  const int b = __builtin_amdgcn_readfirstlane(it[0]);
  const int rg = __builtin_amdgcn_readfirstlane(it[1]);
  const int t0 = __builtin_amdgcn_readfirstlane(it[2]);
  const int t1 = __builtin_amdgcn_readfirstlane(it[3]);
  const int slot = __builtin_amdgcn_readfirstlane(it[4]);
  if (!item_in_range(p, X_RGS, b, rg, t0, t1, slot)) {
    flag_bad_item(p.flags);
    return;
  }

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n32 = lane & 31;
  const int hi = lane >> 5;
  const int L = __builtin_amdgcn_readfirstlane(min(max(p.seq_lens[b], 0), p.max_keys));
  // a cache read by one row group only streams past the caches; with several
  // row groups per sequence the other groups re-read it from L2
  const bool stream_once = p.rows <= X_RGS;

  const int row_local = 32 * w + n32;
  const int row = rg * X_RGS + row_local;
  const bool row_ok = row < p.rows;
  const bool wave_active = rg * X_RGS + 32 * w < p.rows;   // wave-uniform
  int limit = 0;
  if (row_ok) {
    const int tok = row / p.heads;
    const int vis = p.causal ? L - p.s_q + 1 + tok : L;
    limit = min(vis, t1);
  }

  // ---- lane constants (byte offsets) ----
  // K operand (key n32), bf16 k-step t: (slot + kb0) ^ ((t & 3) << 5), plus
  // (t >> 2) * X_GSTRIDE; fp8 k-step pair u: (slot + kb0) ^ ((u & 1) << 5),
  // plus (u >> 1) * X_GSTRIDE + 2048 * (32-key half of the slot)
  // (kb0, computed at each use from a fresh lane id)
  auto kb0_of = [](int ln) -> uint32_t {
    const int n = ln & 31, h = (ln >> 5) & 1;
    if constexpr (!F8)
      return n * 128 + ((h ^ swz16(n)) << 4);
    else
      return n * 64 + (((2 * h) ^ swz8(n)) << 4);
  };
  // V^T operand, bf16 dim block db, 16-key step s, 4-key read x:
  // (slot + vt0) ^ (64 (db & 1) + 32 x), plus (db >> 1) * X_GSTRIDE + 2048 s
  // + 1024 x; fp8: (slot + vt0) ^ (32 (db & 1)), plus (db >> 1) * X_GSTRIDE
  // + 2048 * half + 1024 s (computed at each use from a fresh lane id)
  auto vt0_of = [](int ln) -> uint32_t {
    const int g16 = (ln >> 4) & 1, ig = ln & 15, h = (ln >> 5) & 1;
    if constexpr (!F8) {
      const int j = ig >> 2, r = ig & 3;
      return (4 * h + j) * 128 + (((2 * g16 + (r >> 1)) ^ swz16(4 * h + j)) << 4) + 8 * (r & 1);
    } else {
      const int jj = ig >> 1, q = ig & 1;
      const int key = 4 * h + (jj & 3) + 8 * (jj >> 2);
      return key * 64 + ((g16 ^ swz8(key)) << 4) + 8 * q;
    }
  };

  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const_i32* bt = (const_i32*)(p.block_table + (size_t)b * p.max_blocks);
  // the block size is 64 or 128 (checked on the host): page and row offset
  // are a shift and a mask
  const int bsh = p.bs == 128 ? 7 : 6;
  const int nsteps = (t1 - t0 + X_STEP - 1) / X_STEP;
  const int ntiles = (t1 - t0 + KT - 1) / KT;

  // Issue this wave's X_NDMA transfers of slot-tile j (exactly X_NDMA VMEM
  // instructions; the vmcnt arithmetic relies on it). A tile never crosses a
  // page: items start on 64-key boundaries and pages hold 64 or 128 keys.
  // Lane l of transfer n lands at slot byte n * 1024 + 16 l. bf16: column
  // group n >> 2, key 8(n & 3) + (l >> 3), position l & 7; fp8: column group
  // n >> 2, key 16(n & 3) + (l >> 2), position l & 3. The lane fetches the
  // global chunk that belongs at that position.
  auto issue = [&](int j) {
    const int ts = t0 + KT * j;
    int page = bt[ts >> bsh];
    if (page < 0 || page >= p.num_blocks) page = 0;
    const char* src = reinterpret_cast<const char*>(p.kv) + ((size_t)page * p.bs + (ts & (p.bs - 1))) * ROWB;
    const uint32_t l0 = lds_addr(smem + (j & 3) * X_TILE);
    const int ln = fresh_lane();
    uint32_t dma_lane[2];
    if constexpr (!F8) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = 8 * h + (ln >> 3);   // key bits 1..3 as in transfer parity h
        dma_lane[h] = (ln >> 3) * ROWB + (((ln & 7) ^ swz16(key)) << 4);
      }
    } else {
      dma_lane[0] = dma_lane[1] = (ln >> 2) * ROWB + (((ln & 3) ^ ((ln >> 4) & 3)) << 4);
    }
    auto one = [&](int i, auto nt_tag) {
      const int n = w * X_NDMA + i;
      const char* g = F8 ? src + (n & 3) * 16 * ROWB + (n >> 2) * 64 : src + (n & 3) * 8 * ROWB + (n >> 2) * 128;
      const uint32_t v = F8 ? dma_lane[0] : dma_lane[n & 1];
      if constexpr (decltype(nt_tag)::value)
        lds_dma16_nt(g, v, l0 + n * 1024);
      else
        lds_dma16(g, v, l0 + n * 1024);
    };
    if (stream_once) {
#pragma unroll
      for (int i = 0; i < X_NDMA; ++i) one(i, std::true_type{});
    } else {
#pragma unroll
      for (int i = 0; i < X_NDMA; ++i) one(i, std::false_type{});
    }
  };
  // keys of slot-tile j that hold data; -1 when its page id is out of range
  // (the tile is then zeroed and every key masked)
  auto valid_keys = [&](int j) {
    const int ts = t0 + KT * j;
    int page = bt[ts >> bsh];
    if (page < 0 || page >= p.num_blocks) return -1;
    return min(KT, t1 - ts);
  };
  bool bad_page = false;

  // Tile 0 is requested before q is loaded, so its latency overlaps the q
  // loads (the compiler's own wait for q below also covers it: it was issued
  // first); tile 1 goes out once q is resident, so that wait does not include
  // it while every workgroup starts at once.
  if (ntiles > 0) issue(0);

  // Q^T operand: k-step t holds dims 16t + 8h .. +7 (bf16), or for fp8 (whose
  // K reads take 16 dims per lane at once) 32(t >> 1) + 16h + 8(t & 1) .. +7.
  // Any fixed assignment of dims to k-steps gives the same dot products.
  // k-steps 32..35 (dims 512..575 either way) go to qrope: chunk 2(t - 32) + h
  // of row r at position (2(t - 32) + h) ^ swz16(r) of its 128 bytes. Each
  // wave writes and reads only its own rows.
  // bf16 caches: k-steps 0..31 in registers (qb), 32..35 in qrope.
  // fp8 caches: the 64-dim blocks 0..7 as hi/lo e4m3fn operands in registers
  // (q8h, q8l: lane (row n, half h) byte j is dim 64 blk + 32 h + j, the same
  // bijection as the K operand read below; A and B of the 32x32x64 MFMA pair
  // their bytes by lane half and byte), block 8 (the rope dims) in qrope as
  // chunks 4 part + 2 h + (j >> 4), part 0 = hi, 1 = lo.
  constexpr int QREG = F8 ? 1 : D / 16 - 4;
  bf16x8_t qb[QREG];
  constexpr int Q8 = F8 ? 8 : 1;
  i32x8_t q8h[Q8], q8l[Q8];
  const int qr_off = row_local * 128;
  const int qr_swz = swz16(row_local);
  const uint16_t* qrow_g = p.q + ((size_t)b * p.rows + (row_ok ? row : 0)) * D;
  // fp8: row scale 2^qe puts the row's largest |q| in [128, 256); scores are
  // then sums of products of exact e4m3fn values, and 2^-qe is folded into
  // this row's score scale
  float qmul = 1.f, scale_row = p.scale_log2;
  if constexpr (!F8) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const int d = 16 * t + 8 * hi;
      uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qrow_g + d) : make_uint4(0, 0, 0, 0);
      if (t < QREG)
        qb[t] = __builtin_bit_cast(bf16x8_t, v);
      else
        *reinterpret_cast<uint4*>(qrope + qr_off + (((2 * (t - QREG) + hi) ^ qr_swz) << 4)) = v;
    }
  } else {
    float qmax = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qrow_g + 64 * (c >> 2) + 32 * hi + 8 * (c & 3))
                             : make_uint4(0, 0, 0, 0);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        qmax = fmaxf(qmax, fmaxf(fabsf(__builtin_bit_cast(float, w[i] << 16)),
                                 fabsf(__builtin_bit_cast(float, w[i] & 0xFFFF0000u))));
    }
    qmax = halves_max(qmax);
    const int qe = qmax > 0.f && qmax < INFINITY ? 8 - __builtin_amdgcn_frexp_expf(qmax) : 0;
    qmul = __builtin_ldexpf(1.f, qe);
    scale_row = p.scale_log2 * __builtin_ldexpf(1.f, -qe);
#pragma unroll
    for (int blk = 0; blk < 9; ++blk) {
      uint32_t h8[8], l8[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qrow_g + 64 * blk + 32 * hi + 8 * c)
                               : make_uint4(0, 0, 0, 0);
        split_fp8x8(v, qmul, h8 + 2 * c, l8 + 2 * c);
      }
      if (blk < 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          q8h[blk < Q8 ? blk : 0][i] = static_cast<int>(h8[i]);
          q8l[blk < Q8 ? blk : 0][i] = static_cast<int>(l8[i]);
        }
      } else {
#pragma unroll
        for (int part = 0; part < 2; ++part)
#pragma unroll
          for (int half16 = 0; half16 < 2; ++half16) {
            const uint32_t* src = (part ? l8 : h8) + 4 * half16;
            *reinterpret_cast<uint4*>(qrope + qr_off + (((4 * part + 2 * hi + half16) ^ qr_swz) << 4)) =
                make_uint4(src[0], src[1], src[2], src[3]);
          }
      }
    }
  }
  // q loads (and with them tile 0, issued before) complete here, so the
  // compiler places no wait for them inside the tile loop (it cannot see the
  // DMAs)
  if constexpr (!F8) {
#pragma unroll
    for (int t = 0; t < QREG; ++t) asm volatile("" ::"v"(qb[t]));
  } else {
#pragma unroll
    for (int t = 0; t < Q8; ++t)
#pragma unroll
      // per dword: a 256-bit operand would be an x86 register class in the host pass
      for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(q8h[t][i]), "v"(q8l[t][i]));
  }
  // tile 1 goes out once q and tile 0 are resident
  if (ntiles > 1) issue(1);
  auto q_operand = [&](int t) -> bf16x8_t {
    if (t < QREG) return qb[t];
    return *reinterpret_cast<const bf16x8_t*>(qrope + qr_off + (((2 * (t - QREG) + hi) ^ qr_swz) << 4));
  };
  // The slow loop reads the register part of q from memory at every use, so
  // the q registers die at the fast loop's exit instead of being saved to
  // scratch there for a loop that rarely runs.
  auto q_operand_mem = [&](int t) -> bf16x8_t {
    if (t < QREG) {
      const int d = 16 * t + 8 * hi;
      const uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qrow_g + d) : make_uint4(0, 0, 0, 0);
      return __builtin_bit_cast(bf16x8_t, v);
    }
    return q_operand(t);
  };
  // fp8 operands of block blk: registers (blocks 0..7 in the fast loop),
  // recomputed from memory (blocks 0..7 in the rescaling loop), or qrope
  auto q8_rope = [&](int part) -> i32x8_t {
    const uint4 a = *reinterpret_cast<const uint4*>(qrope + qr_off + (((4 * part + 2 * hi) ^ qr_swz) << 4));
    const uint4 c = *reinterpret_cast<const uint4*>(qrope + qr_off + (((4 * part + 2 * hi + 1) ^ qr_swz) << 4));
    return i32x8_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)c.x, (int)c.y, (int)c.z, (int)c.w};
  };
  auto q8_mem = [&](int blk, i32x8_t& h, i32x8_t& l) {
    uint32_t h8[8], l8[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qrow_g + 64 * blk + 32 * hi + 8 * c)
                             : make_uint4(0, 0, 0, 0);
      split_fp8x8(v, qmul, h8 + 2 * c, l8 + 2 * c);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h[i] = static_cast<int>(h8[i]);
      l[i] = static_cast<int>(l8[i]);
    }
  };

  f32x16_t o[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;


  // The ring runs two tiles ahead. prepare(j) makes tile j resident for
  // every wave (wait for this wave's transfers, zero its slots of keys past
  // the end, barrier), then issues tile j + 2 into the slot of tile j - 2,
  // which every wave has finished with once it is past the barrier: while
  // step k's PV reads tile(k) and step k + 1's QK reads tile(k + 1), the two
  // tiles after them are in flight. Bit (j & 3) of bad_slots records whether
  // tile j's page id was out of range.
  int bad_slots = 0;
  auto prepare = [&](int j) {
    mem_fence_compiler();
    if (j + 1 < ntiles)
      wait_vmcnt<X_NDMA>();
    else
      wait_vmcnt<0>();
    mem_fence_compiler();
    char* t = smem + (j & 3) * X_TILE;
    const int nv = valid_keys(j);
    const bool bad = nv < 0;
    bad_page |= bad;
    bad_slots = (bad_slots & ~(1 << (j & 3))) | (bad ? 1 << (j & 3) : 0);
    if (nv < KT) {
      const int ln = fresh_lane();
      const int lk = F8 ? (ln >> 2) : (ln >> 3);   // key within the transfer
#pragma unroll
      for (int i = 0; i < X_NDMA; ++i) {
        const int n = w * X_NDMA + i;
        if (lk >= nv - (F8 ? 16 : 8) * (n & 3))
          *reinterpret_cast<uint4*>(t + n * 1024 + ln * 16) = make_uint4(0, 0, 0, 0);
      }
    }
    __syncthreads();
    if (j + 2 < ntiles) issue(j + 2);
  };
  auto tile_of = [&](int k) -> const char* { return smem + ((F8 ? k >> 1 : k) & 3) * X_TILE; };
  // Element e of step k's scores (C layout) is a visible key iff
  // 8(e >> 2) + (e & 3) < rel_of(k); a tile whose page id was out of range
  // has none.
  auto rel_of = [&](int k) -> int {
    const int j = F8 ? k >> 1 : k;
    return (bad_slots >> (j & 3)) & 1 ? -64 : limit - (t0 + X_STEP * k) - 4 * hi;
  };

  // S^T of step k (32 keys x this wave's 32 rows) from tile `tile`, with the
  // operands that need no wait states (q from registers or qrope, K from
  // LDS). between(g) runs after the MFMAs of each of the 9 groups of 64 dims:
  // a wave issues in order and an MFMA occupies the matrix core for 32
  // (bf16) or 64 (fp8) cycles, so VALU work placed there executes meanwhile.
  // The K reads are software-pipelined by hand: the asm MFMAs look cheap to
  // the scheduler, which would otherwise issue each read just before its use
  // and expose the LDS latency every time.
  auto qk = [&](const char* tile, int k, f32x16_t& sacc, auto&& between) {
    const uint32_t kbase = lds_addr(tile) + kb0_of(fresh_lane());
    if constexpr (!F8) {
      auto kaddr = [&](int t) { return (kbase ^ ((t & 3) << 5)) + (t >> 2) * X_GSTRIDE; };
      bf16x8_t kr[QK_AHEAD];
#pragma unroll
      for (int t = 0; t < QK_AHEAD; ++t) kr[t] = lds_b128(kaddr(t));
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x8_t a = kr[t % QK_AHEAD];
        if (t + QK_AHEAD < D / 16) kr[t % QK_AHEAD] = lds_b128(kaddr(t + QK_AHEAD));
        if (t == 0)
          qk_first(sacc, a, q_operand(t));
        else
          qk_next(sacc, a, q_operand(t));
        if ((t & 3) == 3) {
          between(t >> 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      // K operand of 64-dim block blk: key 32 half + n32, chunks 2h and
      // 2h + 1 (dims 64 blk + 32 h .. + 31), as stored
      auto kaddr = [&](int blk) { return kbase + blk * X_GSTRIDE + 2048 * (k & 1); };
      auto kread = [&](int blk) -> i32x8_t {
        const u32x4_t a = lds_u128(kaddr(blk)), c = lds_u128(kaddr(blk) ^ 16);
        return i32x8_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
      };
      i32x8_t kr = kread(0);
#pragma unroll
      for (int blk = 0; blk < 9; ++blk) {
        const i32x8_t a = kr;
        if (blk + 1 < 9) kr = kread(blk + 1);
        if (blk == 8) {
          qk8_next(sacc, a, q8_rope(0));
          qk8_next(sacc, a, q8_rope(1));
        } else {
          if (blk == 0)
            qk8_first(sacc, a, q8h[blk]);
          else
            qk8_next(sacc, a, q8h[blk]);
          qk8_next(sacc, a, q8l[blk]);
        }
        between(blk);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto qk_wait = [&](f32x16_t& sacc) {
    if constexpr (F8)
      qk8_done(sacc);
    else
      qk_done(sacc);
  };

  // O^T += V^T P^T over step k's two 16-key halves (tile `tile`): 32 MFMAs,
  // MFMA i on dim block i & 15 of half i >> 4. The V^T reads run PV_AHEAD
  // MFMAs ahead through a ring of raw operands, and the operand of MFMA i + 1
  // is assembled (widened, for fp8) right after MFMA i issues, in its shadow.
  // The order is fixed per MFMA: left to the scheduler, the reads sink to
  // their uses under the loop's register pressure and each MFMA waits for a
  // full LDS round trip.
  auto pv = [&](const char* tile, int k, const bf16x8_t* pb) {
    const int half = F8 ? (k & 1) : 0;   // fp8: which 32 keys of the 64-key slot
    const uint32_t vbase = lds_addr(tile) + vt0_of(fresh_lane());
    constexpr int NPV = 2 * (DV / 32);
    typedef std::conditional_t<F8, uint2, uint4> raw_t;
    auto vread = [&](int i) -> raw_t {
      const int s = i >> 4, db = i & 15;
      if constexpr (!F8) {
        const uint32_t off = (db >> 1) * X_GSTRIDE + 2048 * s;
        const uint2 a0 = __builtin_bit_cast(uint2, lds_tr16((vbase ^ (64 * (db & 1))) + off));
        const uint2 a1 = __builtin_bit_cast(uint2, lds_tr16((vbase ^ (64 * (db & 1) + 32)) + off + 1024));
        return make_uint4(a0.x, a0.y, a1.x, a1.y);
      } else {
        return lds_tr8((vbase ^ (32 * (db & 1))) + (db >> 1) * X_GSTRIDE + 2048 * half + 1024 * s);
      }
    };
    auto operand = [&](const raw_t& r) -> bf16x8_t {
      if constexpr (!F8)
        return __builtin_bit_cast(bf16x8_t, r);
      else
        return __builtin_bit_cast(bf16x8_t, fp8x8_to_bf16x8(r.x, r.y));
    };
    raw_t vr[PV_AHEAD];
#pragma unroll
    for (int i = 0; i < PV_AHEAD; ++i) vr[i] = vread(i);
    bf16x8_t a = operand(vr[0]);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      o[i & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[i >> 4], o[i & 15], 0, 0, 0);
      if (i + PV_AHEAD < NPV) vr[i % PV_AHEAD] = vread(i + PV_AHEAD);
      if (i + 1 < NPV) a = operand(vr[(i + 1) % PV_AHEAD]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Online softmax of one step's raw scores (the scale is folded into the
  // max and the FMA), in 8 stages so that the fast loop can spread it over
  // the next step's QK MFMAs; each stage pins its results (an empty asm that
  // takes them as operands), which keeps the compiler from sinking the work
  // past the QK chain to where it is used. Stage 2 decides whether the step
  // stays on the fast path: no row's max more than BIG_SLACK above its
  // reference (which a row's first keys set). The stages leave m_run, l_run
  // and O alone otherwise; the caller adds lsum to l_run once the step is
  // accepted.
  float sx[16], tmax = 0.f, neg_m = 0.f, lsum = 0.f;
  bool jump = false;
  bf16x8_t pb[2];
  auto pin = [](float& v) { asm volatile("" : "+v"(v)); };
  auto smx = [&](int st, const f32x16_t& sc, int rel) {
    if (st == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sx[e] = sc[e];
      // keys past a row's limit or on a bad page (rare: a uniform branch)
      if (__builtin_amdgcn_ballot_w64(rel < 28)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sx[e] = 8 * (e >> 2) + (e & 3) < rel ? sx[e] : -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) pin(sx[e]);
    } else if (st == 1) {
      tmax = fmaxf(fmaxf(fmaxf(sx[0], sx[1]), fmaxf(sx[2], sx[3])), fmaxf(fmaxf(sx[4], sx[5]), fmaxf(sx[6], sx[7])));
      tmax = fmaxf(tmax, fmaxf(fmaxf(fmaxf(sx[8], sx[9]), fmaxf(sx[10], sx[11])),
                               fmaxf(fmaxf(sx[12], sx[13]), fmaxf(sx[14], sx[15]))));
      pin(tmax);
    } else if (st == 2) {
      tmax = halves_max(tmax) * scale_row;
      if (m_run == -INFINITY) m_run = tmax;   // o and l of this row are still zero
      jump = __builtin_amdgcn_ballot_w64(tmax > m_run + BIG_SLACK) != 0;
      // rows without any key so far keep m = -inf: a finite stand-in makes
      // their masked scores give exp2(-inf) = 0, never NaN
      neg_m = -fmaxf(m_run, -1e30f);
      lsum = 0.f;
      pin(m_run);
      pin(neg_m);
    } else if (st <= 6) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * (st - 3) + i;
        sx[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sx[e], scale_row, neg_m));
        lsum += sx[e];
        pin(sx[e]);
      }
      pin(lsum);
    } else if (st == 7) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        pb[s] = __builtin_bit_cast(
            bf16x8_t, make_uint4(pack_bf16x2(sx[8 * s], sx[8 * s + 1]), pack_bf16x2(sx[8 * s + 2], sx[8 * s + 3]),
                                 pack_bf16x2(sx[8 * s + 4], sx[8 * s + 5]),
                                 pack_bf16x2(sx[8 * s + 6], sx[8 * s + 7])));
        asm volatile("" : "+v"(pb[s]));
      }
    }
  };

  // One step with rescaling (the rare path after a row's max jumped): the q
  // operands are re-read from memory (so q's registers die at the fast
  // loop's exit instead of being saved to scratch for a loop that rarely
  // runs) and reach the MFMAs through VALU code, hence the forms with wait
  // states; every row is rescaled by alpha = 2^(m_old - m_new) (1 for rows
  // whose max did not move: a conditional rescale merges two versions of O
  // and makes the compiler hold all of O in VGPRs).
  auto compute_slow = [&](const char* tile, int k, int rel) {
    f32x16_t sacc;
    const uint32_t kbase = lds_addr(tile) + kb0_of(fresh_lane());
    if constexpr (!F8) {
      auto kaddr = [&](int t) { return (kbase ^ ((t & 3) << 5)) + (t >> 2) * X_GSTRIDE; };
      bf16x8_t kr[QK_AHEAD];
#pragma unroll
      for (int t = 0; t < QK_AHEAD; ++t) kr[t] = lds_b128(kaddr(t));
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x8_t a = kr[t % QK_AHEAD];
        if (t + QK_AHEAD < D / 16) kr[t % QK_AHEAD] = lds_b128(kaddr(t + QK_AHEAD));
        const bf16x8_t qv = q_operand_mem(t);
        if (t == 0)
          qk_first_v(sacc, a, qv);
        else
          qk_next_v(sacc, a, qv);
      }
    } else {
      auto kaddr = [&](int blk) { return kbase + blk * X_GSTRIDE + 2048 * (k & 1); };
      auto kread = [&](int blk) -> i32x8_t {
        const u32x4_t a = lds_u128(kaddr(blk)), c = lds_u128(kaddr(blk) ^ 16);
        return i32x8_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
      };
#pragma unroll
      for (int blk = 0; blk < 9; ++blk) {
        const i32x8_t a = kread(blk);
        i32x8_t h, l;
        if (blk == 8) {
          h = q8_rope(0);
          l = q8_rope(1);
        } else {
          q8_mem(blk, h, l);
        }
        if (blk == 0)
          qk8_first_v(sacc, a, h);
        else
          qk8_next_v(sacc, a, h);
        qk8_next_v(sacc, a, l);
      }
    }
    qk_wait(sacc);
    smx(0, sacc, rel);
    smx(1, sacc, rel);
    tmax = halves_max(tmax) * scale_row;
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);   // m_run = -inf gives 0
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) {
      o[d] *= alpha;
      __builtin_amdgcn_sched_barrier(0);
    }
    neg_m = -fmaxf(m_run, -1e30f);
    lsum = 0.f;
#pragma unroll
    for (int st = 3; st < 8; ++st) smx(st, sacc, rel);
    l_run += lsum;
    __builtin_amdgcn_sched_barrier(0);
    pv(tile, k, pb);
  };

  // Fast loop, software-pipelined across steps: step k + 1's QK MFMAs are
  // interleaved with step k's softmax, then step k's PV follows.
  if (ntiles > 0) prepare(0);
  int k = 0;
  if (!wave_active) {
    // rows past the end: no compute, but the same barriers and transfers
    for (int j = 1; j < ntiles; ++j) prepare(j);
    k = nsteps;
  } else if (nsteps > 0) {
    f32x16_t s_cur;
    int rel_cur = rel_of(0);
    qk(tile_of(0), 0, s_cur, [](int) {});
    qk_wait(s_cur);
    bool jumped = false;
    for (; k + 1 < nsteps; ++k) {
      if (!F8 || (k & 1)) prepare(F8 ? (k + 1) >> 1 : k + 1);
      const int rel_nxt = rel_of(k + 1);
      f32x16_t s_nxt;
      qk(tile_of(k + 1), k + 1, s_nxt, [&](int g) { smx(g, s_cur, rel_cur); });
      // the compiler may move or copy s_nxt (or reuse its registers when the
      // step is dropped) right after the chain: wait for the last MFMA first
      // (its wait states overlap that MFMA's own passes)
      qk_wait(s_nxt);
      if (jump) {
        jumped = true;
        break;
      }
      l_run += lsum;
      pv(tile_of(k), k, pb);
      s_cur = s_nxt;
      rel_cur = rel_nxt;
    }
    if (!jumped) {
#pragma unroll
      for (int g = 0; g < 8; ++g) smx(g, s_cur, rel_cur);
      if (!jump) {
        l_run += lsum;
        pv(tile_of(k), k, pb);
        ++k;
      }
    }
    // rare: finish with rescaling, from step k, whose tile is resident (as
    // is the next step's)
    if (k < nsteps) {
      int prepared = F8 ? min(k + 1, nsteps - 1) >> 1 : min(k + 1, nsteps - 1);
      for (; k < nsteps; ++k) {
        const int j = F8 ? k >> 1 : k;
        if (j > prepared) {
          prepare(j);
          prepared = j;
        }
        compute_slow(tile_of(k), k, rel_of(k));
      }
    }
  }

  flag_bad_page(p.flags, bad_page);

  // ---- write this wave's rows: final (slot < 0) or split partial ----
  // The rows leave through LDS (the ring is free once every wave is past its
  // last step): a wave stages its 32 rows x 256 dims at a time, then writes
  // whole row segments, so each store instruction covers 512 B of one row
  // (bf16 out or fp16 partial) instead of scattered 16-byte pieces.
  // Lane-derived values are derived afresh here, from the lane id, rather
  // than kept from the prologue: kept, they stay live across the tile loop
  // and come back as scratch reloads, each a memory round trip.
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int n32_e = lane_e & 31, hi_e = lane_e >> 5;
  const int row_local_e = 32 * w + n32_e;
  const int row_e = rg * X_RGS + row_local_e;
  const bool row_ok_e = row_e < p.rows;
  const float l_row = halves_sum(l_run);
  const bool empty = !(l_row > 0.f);
  const float inv = empty ? 0.f : p.out_scale / l_row;
  const float lse2 = empty ? -INFINITY : m_run + log2f(l_row);
  // A split partial row leaves as fp16 o * 2^k (partial_exponent). Here 2^k
  // is folded into the normalisation factor, with k capped so that inv * 2^k
  // stays finite (which only matters for rows whose values are all far below
  // 2^-100).
  int kexp = 0;
  if (slot >= 0) {
    float amax = 0.f;
#pragma unroll
    for (int db = 0; db < DV / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(o[db][e]));
    amax = halves_max(amax) * inv;   // this row's largest |o| after normalisation
    kexp = min(partial_exponent(amax), 127 - __builtin_amdgcn_frexp_expf(inv));
  }
  const float fs = __builtin_ldexpf(inv, kexp);   // normalisation and 2^k in one factor
  if (row_ok_e && hi_e == 0) {
    if (slot < 0) {
      if (p.lse != nullptr) p.lse[(size_t)b * p.rows + row_e] = lse2 * LN2;
    } else {
      p.part_lse[(size_t)slot * X_RGS + row_local_e] = lse2;
      p.part_scale[(size_t)slot * X_RGS + row_local_e] = kexp;
    }
  }
  __syncthreads();   // every wave is done with the ring
  constexpr int SROW = 260;   // floats per staged row: 256 + 4 (rows 16 bytes apart in the banks)
  static_assert(4 * 32 * SROW * 4 <= X_SLOTS * X_TILE, "staging fits in the ring");
  float* stage = reinterpret_cast<float*>(smem) + w * 32 * SROW;
  const int nrow = min(32, p.rows - (rg * X_RGS + 32 * w));   // this wave's valid rows (wave-uniform)
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int db = 0; db < DV / 64; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x16_t& a = o[(DV / 64) * hf + db];
        *reinterpret_cast<f32x4_t*>(stage + n32_e * SROW + 32 * db + 8 * q + 4 * hi_e) =
            f32x4_t{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]} * fs;
      }
    // a wave's LDS accesses complete in order: the reads below see the writes
    for (int r = 0; r < nrow; ++r) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stage + r * SROW + 4 * lane_e);
      const int rl = 32 * w + r;
      if (slot < 0) {
        uint16_t* dst = p.out + ((size_t)b * p.rows + rg * X_RGS + rl) * DV + (DV / 2) * hf + 4 * lane_e;
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      } else {
        _Float16* dst = p.part_o + ((size_t)slot * X_RGS + rl) * DV + (DV / 2) * hf + 4 * lane_e;
        *reinterpret_cast<f16x4_t*>(dst) = __builtin_convertvector(v, f16x4_t);
      }
    }
  }
}

}  // namespace

namespace mla_detail {

void launch_wide128(int kv_dtype, dim3 grid, hipStream_t st, const FwdParams& fp) {
  if (kv_dtype == MLA_DTYPE_BF16)
    hipLaunchKernelGGL((mla_decode_wide128<MLA_DTYPE_BF16>), grid, dim3(NTHREADS), 0, st, fp);
  else
    hipLaunchKernelGGL((mla_decode_wide128<MLA_DTYPE_FP8_E4M3FN>), grid, dim3(NTHREADS), 0, st, fp);
}

}  // namespace mla_detail
