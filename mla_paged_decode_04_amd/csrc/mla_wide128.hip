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
#define PV_AHEAD 4                // PV MFMAs whose V^T reads are issued ahead
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
typedef int i32x8_t __attribute__((ext_vector_type(8)));
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

// Four float32 values x (|x| < 256) -> e4m3fn codes of hi = nearest(x) and
// lo = nearest(x - hi), packed four to a dword. For x = q * 2^e with q a bf16
// value (8 significant bits) the residual x - hi is a multiple of q's last
// place with at most 4 significant bits, so lo is exact and hi + lo = x
// whenever that place is at least e4m3fn's smallest step 2^-9 (elements down
// to 2^-10 of a row maximum scaled to [128, 256); smaller ones lose bits
// below 2^-18 of the row maximum).
typedef short s16x2_t __attribute__((ext_vector_type(2)));
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
  const int n_items = p.header[0];
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
  // DMA: lane l of transfer n lands at slot byte n * 1024 + 16 l. bf16:
  // column group n >> 2, key 8(n & 3) + (l >> 3), position l & 7; fp8: column
  // group n >> 2, key 16(n & 3) + (l >> 2), position l & 3. The lane fetches
  // the global chunk that belongs at that position.
  uint32_t dma_lane[2];
  // K operand (key n32), bf16 k-step t: (slot + kb0) ^ ((t & 3) << 5), plus
  // (t >> 2) * X_GSTRIDE; fp8 k-step pair u: (slot + kb0) ^ ((u & 1) << 5),
  // plus (u >> 1) * X_GSTRIDE + 2048 * (32-key half of the slot)
  uint32_t kb0;
  // V^T operand, bf16 dim block db, 16-key step s, 4-key read x:
  // (slot + vt0) ^ (64 (db & 1) + 32 x), plus (db >> 1) * X_GSTRIDE + 2048 s
  // + 1024 x; fp8: (slot + vt0) ^ (32 (db & 1)), plus (db >> 1) * X_GSTRIDE
  // + 2048 * half + 1024 s
  uint32_t vt0;
  {
    const int g16 = (lane >> 4) & 1, ig = lane & 15;
    if constexpr (!F8) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = 8 * h + (lane >> 3);   // key bits 1..3 as in transfer parity h
        dma_lane[h] = (lane >> 3) * ROWB + (((lane & 7) ^ swz16(key)) << 4);
      }
      kb0 = n32 * 128 + ((hi ^ swz16(n32)) << 4);
      const int j = ig >> 2, r = ig & 3;
      vt0 = (4 * hi + j) * 128 + (((2 * g16 + (r >> 1)) ^ swz16(4 * hi + j)) << 4) + 8 * (r & 1);
    } else {
      dma_lane[0] = dma_lane[1] = (lane >> 2) * ROWB + (((lane & 3) ^ ((lane >> 4) & 3)) << 4);
      kb0 = n32 * 64 + (((2 * hi) ^ swz8(n32)) << 4);
      const int jj = ig >> 1, q = ig & 1;
      const int key = 4 * hi + (jj & 3) + 8 * (jj >> 2);
      vt0 = key * 64 + ((g16 ^ swz8(key)) << 4) + 8 * q;
    }
  }

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
  auto issue = [&](int j) {
    const int ts = t0 + KT * j;
    int page = bt[ts >> bsh];
    if (page < 0 || page >= p.num_blocks) page = 0;
    const char* src = reinterpret_cast<const char*>(p.kv) + ((size_t)page * p.bs + (ts & (p.bs - 1))) * ROWB;
    const uint32_t l0 = lds_addr(smem + (j & 3) * X_TILE);
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
  bool bad_page = false, tile_bad = false;

  // Tile 0 is requested before q is loaded, so its latency overlaps the q
  // loads (the compiler's own wait for q below also covers it: it was issued
  // first); tiles 1 and 2 go out once q is resident, so that wait does not
  // include them while every workgroup starts at once.
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
  // tiles 1 and 2 go out once q and tile 0 are resident
#pragma unroll
  for (int k = 1; k < 3; ++k)
    if (k < ntiles) issue(k);
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


  // Make slot-tile j resident for every wave: wait for this wave's transfers,
  // zero its slots of keys past the end, barrier (tile j complete everywhere;
  // tile j - 1 consumed by every wave), then issue tile j + 3 into the slot
  // of tile j - 1.
  auto prepare = [&](int j) -> const char* {
    mem_fence_compiler();
    const int ahead = min(2, ntiles - 1 - j);
    if (ahead >= 2)
      wait_vmcnt<2 * X_NDMA>();
    else if (ahead == 1)
      wait_vmcnt<X_NDMA>();
    else
      wait_vmcnt<0>();
    mem_fence_compiler();
    char* cur = smem + (j & 3) * X_TILE;
    const int nv = valid_keys(j);
    tile_bad = nv < 0;
    bad_page |= tile_bad;
    if (nv < KT) {
      const int lk = F8 ? (lane >> 2) : (lane >> 3);   // key within the transfer
#pragma unroll
      for (int i = 0; i < X_NDMA; ++i) {
        const int n = w * X_NDMA + i;
        if (lk >= nv - (F8 ? 16 : 8) * (n & 3))
          *reinterpret_cast<uint4*>(cur + n * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
      }
    }
    __syncthreads();
    if (j + 3 < ntiles) issue(j + 3);
    return cur;
  };

  // One 32-key step k (slot-tile cur). The fast variant never touches the
  // accumulators with VALU code and returns false (before consuming the
  // step) if a row's max jumped more than BIG_SLACK above its reference.
  auto compute = [&](const char* cur, int k, auto slow_tag) -> bool {
    constexpr bool SLOW = decltype(slow_tag)::value;
    if (!wave_active) return true;
    const int ts = t0 + X_STEP * k;
    const int half = F8 ? (k & 1) : 0;   // fp8: which 32 keys of the 64-key slot

    // ---- S^T: 32 keys x this wave's 32 rows ----
    // The K reads are software-pipelined QK_AHEAD k-steps ahead by hand: the
    // asm MFMAs look cheap to the scheduler, which would otherwise issue each
    // read just before its use and expose the LDS latency on every k-step.
    f32x16_t sacc;
    const uint32_t kbase = lds_addr(cur) + kb0;
    if constexpr (!F8) {
      auto kaddr = [&](int t) { return (kbase ^ ((t & 3) << 5)) + (t >> 2) * X_GSTRIDE; };
      bf16x8_t kr[QK_AHEAD];
#pragma unroll
      for (int t = 0; t < QK_AHEAD; ++t) kr[t] = lds_b128(kaddr(t));
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x8_t a = kr[t % QK_AHEAD];
        if (t + QK_AHEAD < D / 16) kr[t % QK_AHEAD] = lds_b128(kaddr(t + QK_AHEAD));
        // the rescaling loop's q operand comes through a VALU select
        // (masked rows), so it takes the forms with the wait states
        if constexpr (SLOW) {
          const bf16x8_t qv = q_operand_mem(t);
          if (t == 0)
            qk_first_v(sacc, a, qv);
          else
            qk_next_v(sacc, a, qv);
        } else {
          const bf16x8_t qv = q_operand(t);
          if (t == 0)
            qk_first(sacc, a, qv);
          else
            qk_next(sacc, a, qv);
        }
      }
    } else {
      // K operand of 64-dim block blk: key 32 half + n32, chunks 2h and
      // 2h + 1 (dims 64 blk + 32 h .. + 31), no conversion
      auto kaddr = [&](int blk) { return kbase + blk * X_GSTRIDE + 2048 * half; };
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
          const i32x8_t h = q8_rope(0), l = q8_rope(1);
          qk8_next(sacc, a, h);
          qk8_next(sacc, a, l);
        } else if constexpr (SLOW) {
          // operands recomputed with VALU code: the forms with wait states
          i32x8_t h, l;
          q8_mem(blk, h, l);
          if (blk == 0)
            qk8_first_v(sacc, a, h);
          else
            qk8_next_v(sacc, a, h);
          qk8_next_v(sacc, a, l);
        } else {
          if (blk == 0)
            qk8_first(sacc, a, q8h[blk]);
          else
            qk8_next(sacc, a, q8h[blk]);
          qk8_next(sacc, a, q8l[blk]);
        }
      }
    }
    if constexpr (F8)
      qk8_done(sacc);
    else
      qk_done(sacc);

    // ---- online softmax on the raw scores (scale folded into max and FMA) ----
    float x[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = sacc[e];
    // a step that reaches a row's limit, or whose page id was out of range
    if (tile_bad || __builtin_amdgcn_ballot_w64(ts + X_STEP > limit)) {
      // element e is visible iff 8(e >> 2) + (e & 3) < rel
      const int rel = tile_bad ? -64 : limit - ts - 4 * hi;
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = 8 * (e >> 2) + (e & 3) < rel ? x[e] : -INFINITY;
    }
    float tmax = x[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, x[e]);
    tmax = halves_max(tmax) * scale_row;
    if constexpr (!SLOW) {
      if (m_run == -INFINITY) m_run = tmax;   // o and l of this row are still zero
      if (__builtin_amdgcn_ballot_w64(tmax > m_run + BIG_SLACK)) return false;
    } else {
      // unconditional (alpha = 1 for rows whose max did not move): a
      // conditional rescale merges two versions of O and makes the compiler
      // hold all of O in VGPRs; one block at a time needs 16 temporaries
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);   // m_run = -inf gives 0
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DV / 32; ++d) {
        o[d] *= alpha;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // rows without any key so far keep m = -inf: a finite stand-in makes
    // their masked scores give exp2(-inf) = 0, never NaN
    const float neg_m = -fmaxf(m_run, -1e30f);
    float pe[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], scale_row, neg_m));
      l_run += pe[e];
    }
    bf16x8_t pb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
      pb[s] = __builtin_bit_cast(
          bf16x8_t, make_uint4(pack_bf16x2(pe[8 * s], pe[8 * s + 1]), pack_bf16x2(pe[8 * s + 2], pe[8 * s + 3]),
                               pack_bf16x2(pe[8 * s + 4], pe[8 * s + 5]), pack_bf16x2(pe[8 * s + 6], pe[8 * s + 7])));

    // keep the V^T reads of the PV loop out of the softmax code above (their
    // registers would stay live across it)
    __builtin_amdgcn_sched_barrier(0);
    // ---- O^T += V^T P^T over the two 16-key steps ----
    const uint32_t vbase = lds_addr(cur) + vt0;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int db = 0; db < DV / 32; ++db) {
        bf16x8_t a;
        if constexpr (!F8) {
          const uint32_t off = (db >> 1) * X_GSTRIDE + 2048 * s;
          const s16x4_t a0 = lds_tr16((vbase ^ (64 * (db & 1))) + off);
          const s16x4_t a1 = lds_tr16((vbase ^ (64 * (db & 1) + 32)) + off + 1024);
          a = __builtin_bit_cast(
              bf16x8_t, make_uint4(__builtin_bit_cast(uint2, a0).x, __builtin_bit_cast(uint2, a0).y,
                                   __builtin_bit_cast(uint2, a1).x, __builtin_bit_cast(uint2, a1).y));
        } else {
          const uint2 v = lds_tr8((vbase ^ (32 * (db & 1))) + (db >> 1) * X_GSTRIDE + 2048 * half + 1024 * s);
          a = __builtin_bit_cast(bf16x8_t, fp8x8_to_bf16x8(v.x, v.y));
        }
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s], o[db], 0, 0, 0);
      }
    }
    // Interleave the PV reads and MFMAs with a bounded read-ahead: left to
    // itself the scheduler issues nearly all 64 reads first, and the
    // registers they hold push the loop's lane constants out to scratch.
    {
      constexpr int RPM = F8 ? 1 : 2;   // LDS reads per MFMA
#pragma unroll
      for (int i = 0; i < PV_AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
#pragma unroll
      for (int i = 0; i < 2 * (DV / 32) - PV_AHEAD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
      }
#pragma unroll
      for (int i = 0; i < PV_AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    return true;
  };

  int k = 0;
  const char* cur = nullptr;
  for (; k < nsteps; ++k) {
    if (!F8 || (k & 1) == 0) cur = prepare(F8 ? (k >> 1) : k);
    if (!compute(cur, k, std::false_type{})) break;
  }
  if (k < nsteps) {   // rare: finish with rescaling, starting at the resident step k
    compute(cur, k, std::true_type{});
    for (++k; k < nsteps; ++k) {
      if (!F8 || (k & 1) == 0) cur = prepare(F8 ? (k >> 1) : k);
      compute(cur, k, std::true_type{});
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
