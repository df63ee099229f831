// Paged MLA decode, > 64 query rows per sequence (the 128-head cases):
// decode attention of MLA in its MQA form ("[WIP][Attention] FlashAttn MLA",
// description) with 128 query rows per work item on 8 waves of 16 rows, two
// waves per SIMD. A wave's output rows (16 x 512 fp32) take 128 registers,
// which leaves room for a second wave on every SIMD: while one wave waits for
// LDS or runs its softmax, the other keeps the matrix core busy. All 8 waves
// share the key tiles streamed HBM -> LDS. With fp8 e4m3fn caches
// ("[Attention] Blackwell FP8 MLA support with CUTLASS_MLA backend", Test
// Plan) the scores run on the 16x16x128 fp8 MFMA against an exact two-term
// fp8 split of q, and V is widened to bf16 in registers before each PV MFMA.
#include <type_traits>

#include "mla_internal.h"

using namespace mla_detail;

namespace {

constexpr int Y_WAVES = 8;
constexpr int Y_THREADS = 64 * Y_WAVES;
constexpr int Y_RGS = 16 * Y_WAVES;   // query rows per work item
constexpr int Y_SLOT = 36864;         // ring slot: 32 bf16 keys or 64 fp8 keys of 576 dims
constexpr int Y_SLOTS = 4;            // three slots in flight while one is computed
constexpr int Y_DMA_WAVES = 4;        // waves 0-3 issue a slot's 36 transfers
constexpr int Y_NDMA = 9;             // 1 KB transfers per DMA wave per slot
constexpr int BF_GS = 32 * 128;       // bf16 slot: bytes per 128-byte column group
constexpr int F8_TILE = 32 * D;       // fp8 slot: two tiles of 32 keys
constexpr int F8_GS = 32 * 64;        // fp8 tile: bytes per 64-byte column group
#ifndef KV_AHEAD
#define KV_AHEAD 4                    // K (QK) and V^T (PV) operand reads kept in flight
#endif

// fp8 tile layout: [9 column groups of 64 B][32 keys][4 x 16 B chunks], chunk
// c of key k at position c ^ swz8(k), swz8(k) = k bit 2 + 2 * k bit 4. With
// it the K reads (16 bytes per lane, keys 16 mi + (lane & 15)) and the
// transposed V reads (8 bytes per lane, keys 4g + 0..3 and 16 + 4g + 0..3)
// are free of LDS bank conflicts; the earlier swizzle ((k >> 2) + (k >> 4)) & 3
// doubled the LDS cycles of both (measured on MI355X with the bank-conflict
// counter on each access pattern in isolation).
__device__ __forceinline__ int swz8(int key) { return ((key >> 2) & 1) | (((key >> 4) & 1) << 1); }

// Max over the four 16-lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48) with
// gfx950's row-swap permutes, issued from inline asm (through the builtins
// the compiler folds max(swap result 0, swap result 1) to result 0).
__device__ __forceinline__ float max4_groups(float v) {
  float y = v;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(v), "+v"(y));
  v = fmaxf(v, y);
  y = v;
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(v), "+v"(y));
  return fmaxf(v, y);
}

// The lane id, read afresh where it is used: an opaque asm the compiler can
// neither merge with other reads nor hoist out of the loop. Lane constants
// derived from it are recomputed at each use (a few VALU instructions)
// rather than kept live across the tile loop, where the register pressure
// would send them to scratch, and the wait for a scratch reload would also
// wait for every tile transfer in flight.
__device__ __forceinline__ int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t lds_u128(const char* a) {
  return *reinterpret_cast<const u32x4_t*>(a);
}
__device__ __forceinline__ uint2 lds_tr8(const char* a) {
  return __builtin_bit_cast(
      uint2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(a)));
}

// MFMA operand layouts (16x16, k = 32 bf16 or 128 fp8 per lane group):
// A[m][k] and B[k][n] put m (or n) = lane & 15 and k = (k per lane) * (lane
// >> 4) + i in element i; C[m][n] puts n = lane & 15 and m = 4 (lane >> 4) + e.
//   S^T (16 keys x 16 rows) = K (A, from LDS) . Q^T (B, registers)
//   O^T (16 dims x 16 rows) += V^T (A, transposed LDS reads) . P^T (B)
// Lane (row c16, group g) thus holds the scores of keys 4g + e of each 16-key
// block, and P^T's k-slot 8g + i is key 4g + i (i < 4) of block 0 or
// 16 + 4g + i - 4 of block 1; the V^T reads deliver the same key order.
template <int KVT>
__global__ __launch_bounds__(Y_THREADS, 1) void mla_decode_wide128(FwdParams p) {
  constexpr bool F8 = KVT == MLA_DTYPE_FP8_E4M3FN;
  constexpr int KT = F8 ? 64 : 32;       // keys per ring slot
  constexpr int ROWB = F8 ? D : 2 * D;   // bytes per cached row
  constexpr int R = KV_AHEAD;
  __shared__ __attribute__((aligned(1024))) char smem[Y_SLOTS * Y_SLOT];   // 147456 bytes
  // the rope part of q, per wave in its operand layout (2 KB per wave)
  __shared__ __attribute__((aligned(1024))) char qlds[Y_WAVES * 2048];     // 16384 bytes

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
  if (!item_in_range(p, Y_RGS, b, rg, t0, t1, slot)) {
    flag_bad_item(p.flags);
    return;
  }

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int L = __builtin_amdgcn_readfirstlane(min(max(p.seq_lens[b], 0), p.max_keys));
  // a cache read by one row group only streams past the caches; with several
  // row groups per sequence the other groups re-read it from L2
  const bool stream_once = p.rows <= Y_RGS;
  const bool dma_wave = w < Y_DMA_WAVES;

  const int row_local = 16 * w + c16;
  const int row = rg * Y_RGS + row_local;
  const bool row_ok = row < p.rows;
  const bool wave_active = rg * Y_RGS + 16 * w < p.rows;   // wave-uniform
  int limit = 0;
  if (row_ok) {
    const int tok = row / p.heads;
    const int vis = p.causal ? L - p.s_q + 1 + tok : L;
    limit = min(vis, t1);
  }

  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const_i32* bt = (const_i32*)(p.block_table + (size_t)b * p.max_blocks);
  // the block size is 64 or 128 (checked on the host): page and row offset
  // are a shift and a mask; a slot never crosses a page (items start on
  // 64-key boundaries)
  const int bsh = p.bs == 128 ? 7 : 6;
  const int ntiles = (t1 - t0 + KT - 1) / KT;

  // Issue this wave's Y_NDMA transfers of slot j (DMA waves only; exactly
  // Y_NDMA VMEM instructions, which the vmcnt arithmetic relies on). Lane l
  // of transfer n lands at slot byte n * 1024 + 16 l.
  // bf16: transfer n = column group n >> 2, key 8 (n & 3) + (l >> 3),
  //   position l & 7 of the key's 8 chunks (chunk c sits at c ^ (key & 7)).
  // fp8: transfers 0-17 fill the tile of keys 0-31, 18-35 that of keys 32-63;
  //   transfer m of a tile = column group m >> 1, key 16 (m & 1) + (l >> 2),
  //   position l & 3 (chunk c at c ^ swz8(key)).
  // The lane fetches the global chunk that belongs at its position.
  auto issue = [&](int j) {
    const int ts = t0 + KT * j;
    int page = bt[ts >> bsh];
    if (page < 0 || page >= p.num_blocks) page = 0;
    const char* src = reinterpret_cast<const char*>(p.kv) + ((size_t)page * p.bs + (ts & (p.bs - 1))) * ROWB;
    const uint32_t l0 = lds_addr(smem + (j & 3) * Y_SLOT);
    const int ln = fresh_lane();
    auto all = [&](auto nt_tag) {
      auto one = [&](const char* gsrc, uint32_t voff, uint32_t lds) {
        if constexpr (decltype(nt_tag)::value)
          lds_dma16_nt(gsrc, voff, lds);
        else
          lds_dma16(gsrc, voff, lds);
      };
      if constexpr (!F8) {
        const uint32_t dl = (ln >> 3) * ROWB + (((ln & 7) ^ (ln >> 3)) << 4);
#pragma unroll
        for (int i = 0; i < Y_NDMA; ++i) {
          const int n = Y_NDMA * w + i;
          one(src + (n & 3) * 8 * ROWB + (n >> 2) * 128, dl, l0 + n * 1024);
        }
      } else {
        const int th = w >> 1;   // which 32-key tile of the slot this wave fills
        const char* s2 = src + th * 32 * ROWB;
        const uint32_t l2 = l0 + th * F8_TILE;
        // transfer m's key half h = m & 1 alternates with i; wave parity
        // decides the phase
        uint32_t dl[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          dl[h] = (ln >> 2) * ROWB + (((ln & 3) ^ (((ln >> 4) & 1) | (2 * h))) << 4);
        const bool odd = w & 1;
#pragma unroll
        for (int i = 0; i < Y_NDMA; ++i) {
          const int m = Y_NDMA * (w & 1) + i;
          const uint32_t voff = odd ? dl[(i + 1) & 1] : dl[i & 1];
          one(s2 + (m & 1) * 16 * ROWB + (m >> 1) * 64, voff, l2 + m * 1024);
        }
      }
    };
    if (stream_once)
      all(std::true_type{});
    else
      all(std::false_type{});
  };
  // keys of slot j that hold data; -1 when its page id is out of range (the
  // slot is then zeroed and every key masked)
  auto valid_keys = [&](int j) {
    const int ts = t0 + KT * j;
    int page = bt[ts >> bsh];
    if (page < 0 || page >= p.num_blocks) return -1;
    return min(KT, t1 - ts);
  };
  bool bad_page = false, tile_bad = false;

  // Slot 0 is requested before q is loaded, so the compiler's own wait for
  // the q loads (it cannot see the DMAs) also covers it; slots 1 and 2 go
  // out behind the q loads (bf16) or once q is converted (fp8).
  if (dma_wave && ntiles > 0) issue(0);

  // ---- q operands ----
  // bf16: qb[s] = dims 32 s + 8 g .. +7 of this lane's row for s < 16; the
  // rope steps s = 16, 17 sit in qlds at (s - 16) * 1024 + 16 lane.
  // fp8: the row q * 2^qe (largest |q| in [128, 256)) split into e4m3fn hi +
  // lo codes; q8h/q8l[s] = dims 128 s + 32 g .. +31 for s < 4; the rope
  // operand (dims 512 + 32 (g & 1) .. +31 as hi codes for g < 2, lo codes for
  // g >= 2, so one MFMA takes both terms) sits in qlds as two 16-byte halves
  // at hh * 1024 + 16 lane.
  constexpr int QB = F8 ? 1 : 16;
  bf16x8_t qb[QB];
  i32x8_t q8h[F8 ? 4 : 1], q8l[F8 ? 4 : 1];
  char* const qw = qlds + w * 2048;
  float scale_row = p.scale_log2;   // fp8: times 2^-qe
  const uint16_t* qrow = p.q + ((size_t)b * p.rows + (row_ok ? row : 0)) * D;
  if constexpr (!F8) {
    // slots 1 and 2 go out right behind the q loads, so the memory pipe
    // stays full while q lands; the wait for q then covers them too (in
    // order), and the first steps find their tiles resident (3 % at 64 x
    // 128 heads, 1-2k keys). The fp8 path requests them after its q
    // conversion instead, which overlaps their arrival.
    uint4 v[18];
#pragma unroll
    for (int s = 0; s < 18; ++s) v[s] = load16_masked(qrow + 32 * s + 8 * g, row_ok);
    __builtin_amdgcn_sched_barrier(0);
    if (dma_wave) {
      if (ntiles > 1) issue(1);
      if (ntiles > 2) issue(2);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 18; ++s) {
      if (s < 16)
        qb[s < 16 ? s : 0] = __builtin_bit_cast(bf16x8_t, v[s]);
      else
        *reinterpret_cast<uint4*>(qw + (s - 16) * 1024 + 16 * lane) = v[s];
    }
#pragma unroll
    for (int s = 0; s < QB; ++s) asm volatile("" ::"v"(qb[s]));
  } else {
    uint4 v[5][4];
    float qmax = 0.f;
    // all 20 loads first: one memory round trip (interleaved with the max
    // below, the scheduler spreads them over several)
#pragma unroll
    for (int s = 0; s < 5; ++s)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        v[s][c] = load16_masked(qrow + (s < 4 ? 128 * s + 32 * g + 8 * c : 512 + 32 * (g & 1) + 8 * c), row_ok);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 5; ++s)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t w4[4] = {v[s][c].x, v[s][c].y, v[s][c].z, v[s][c].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          qmax = fmaxf(qmax, fmaxf(fabsf(__builtin_bit_cast(float, w4[i] << 16)),
                                   fabsf(__builtin_bit_cast(float, w4[i] & 0xFFFF0000u))));
      }
    qmax = wave_max_across_groups(qmax);
    const int qe = qmax > 0.f && qmax < INFINITY ? 8 - __builtin_amdgcn_frexp_expf(qmax) : 0;
    const float qmul = __builtin_ldexpf(1.f, qe);
    scale_row = p.scale_log2 * __builtin_ldexpf(1.f, -qe);
#pragma unroll
    for (int s = 0; s < 5; ++s) {
      uint32_t h8[8], l8[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) split_fp8x8(v[s][c], qmul, h8 + 2 * c, l8 + 2 * c);
      if (s < 4) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          q8h[s < 4 ? s : 0][i] = static_cast<int>(h8[i]);
          q8l[s < 4 ? s : 0][i] = static_cast<int>(l8[i]);
        }
      } else {
        const uint32_t* r = g < 2 ? h8 : l8;
        *reinterpret_cast<uint4*>(qw + 16 * lane) = make_uint4(r[0], r[1], r[2], r[3]);
        *reinterpret_cast<uint4*>(qw + 1024 + 16 * lane) = make_uint4(r[4], r[5], r[6], r[7]);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      // per dword: a 256-bit operand would be an x86 register class in the host pass
      for (int s = 0; s < 4; ++s) asm volatile("" ::"v"(q8h[s][i]), "v"(q8l[s][i]));
  }
  if (F8 && dma_wave) {
    if (ntiles > 1) issue(1);
    if (ntiles > 2) issue(2);
  }

  f32x4_t o[DV / 16];
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- lane operand offsets inside a tile ----
  // K, bf16: key 16 mi + c16, dims 32 s + 8 g: chunk 4 (s & 1) + g of column
  //   group s >> 1; fp8: key 16 mi + c16, bytes 32 g .. +31 of 128-dim step s:
  //   column group 2 s + (g >> 1), chunks 2 (g & 1) + h (h = 0, 1); the rope
  //   step reads column group 8 for every g.
  // V^T, bf16: two 4-key transposed reads per 16 dims; fp8: one 8-key read.
  // (computed from a fresh lane id at each use, see fresh_lane)
  auto k_offsets = [](int ln, int (&kb)[2][2]) {
    const int c = ln & 15, gg = ln >> 4;
    if constexpr (!F8) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int par = 0; par < 2; ++par) kb[mi][par] = (16 * mi + c) * 128 + (((4 * par + gg) ^ (c & 7)) << 4);
    } else {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          kb[mi][h] = (16 * mi + c) * 64 + (((2 * (gg & 1) + h) ^ swz8(16 * mi + c)) << 4);
    }
  };
  auto v_offsets = [](int ln, int (&vt)[4]) {
    const int c = ln & 15, gg = ln >> 4;
    if constexpr (!F8) {
      const int j = c >> 2, q = c & 3;
      const int lanex = (q >> 1) ^ ((gg & 1) << 2) ^ j;
#pragma unroll
      for (int x = 0; x < 4; ++x) vt[x] = (4 * gg + j) * 128 + (((2 * x) ^ lanex) << 4) + (q & 1) * 8;
    } else {
      const int jj = c >> 1, q = c & 1;
      const int key = jj < 4 ? 4 * gg + jj : 16 + 4 * gg + (jj - 4);
#pragma unroll
      for (int x = 0; x < 4; ++x) vt[x] = key * 64 + ((x ^ swz8(key)) << 4) + q * 8;
    }
  };

  // S^T of 32 keys (two 16-key blocks) x this wave's 16 rows, with the K
  // operand reads kept R MFMAs ahead of their use.
  auto qk = [&](const char* tile, f32x4_t (&sacc)[2]) {
    const int ln = fresh_lane();
    int kb[2][2];
    k_offsets(ln, kb);
    if constexpr (!F8) {
      constexpr int N = 36;   // MFMA i: k-step i >> 1, block i & 1
      auto kread = [&](int i) -> bf16x8_t {
        const int s = i >> 1, mi = i & 1;
        return *reinterpret_cast<const bf16x8_t*>(tile + kb[mi][s & 1] + (s >> 1) * BF_GS);
      };
      bf16x8_t kr[R];
#pragma unroll
      for (int i = 0; i < R; ++i) kr[i] = kread(i);
      bf16x8_t qr[2];
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const bf16x8_t a = kr[i % R];
        if (i + R < N) kr[i % R] = kread(i + R);
        if (i == 24) {
          qr[0] = *reinterpret_cast<const bf16x8_t*>(qw + 16 * ln);
          qr[1] = *reinterpret_cast<const bf16x8_t*>(qw + 1024 + 16 * ln);
        }
        const int s = i >> 1;
        const bf16x8_t bq = s < 16 ? qb[s < 16 ? s : 0] : qr[s - 16 < 0 ? 0 : s - 16];
        sacc[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq, i < 2 ? f32x4_t{0.f, 0.f, 0.f, 0.f}
                                                                           : sacc[i & 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // read pair i (two 16-byte chunks): 128-dim step i >> 1 (4 = rope), block i & 1
      constexpr int N = 10;
      constexpr int R8 = R / 2 > 0 ? R / 2 : 1;
      const char* kg = tile + ((ln >> 5) & 1) * F8_GS;
      auto kread = [&](int i) -> i32x8_t {
        const int s = i >> 1, mi = i & 1;
        const char* base = s < 4 ? kg + 2 * s * F8_GS : tile + 8 * F8_GS;
        const u32x4_t x = lds_u128(base + kb[mi][0]), y = lds_u128(base + kb[mi][1]);
        return i32x8_t{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
      };
      i32x8_t kr[R8];
#pragma unroll
      for (int i = 0; i < R8; ++i) kr[i] = kread(i);
      i32x8_t qr;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const i32x8_t a = kr[i % R8];
        if (i + R8 < N) kr[i % R8] = kread(i + R8);
        if (i == 6) {
          const u32x4_t x = lds_u128(qw + 16 * ln), y = lds_u128(qw + 1024 + 16 * ln);
          qr = i32x8_t{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
        }
        const int s = i >> 1, mi = i & 1;
        if (s < 4) {
          sacc[mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a, q8h[s < 4 ? s : 0], s == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : sacc[mi], 0, 0, 0, 0, 0, 0);
          sacc[mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, q8l[s < 4 ? s : 0], sacc[mi], 0, 0, 0, 0,
                                                                      0, 0);
        } else {
          sacc[mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qr, sacc[mi], 0, 0, 0, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // O^T += V^T P^T over 32 keys: 32 MFMAs (16 dims each), the V^T reads R
  // MFMAs ahead; an fp8 operand is widened right after the previous MFMA
  // issues.
  auto pv = [&](const char* tile, const bf16x8_t& pb) {
    int vt[4];
    v_offsets(fresh_lane(), vt);
    if constexpr (!F8) {
      auto vread = [&](int dt) -> uint4 {
        const char* src = tile + vt[dt & 3] + (dt >> 2) * BF_GS;
        const uint2 a0 = __builtin_bit_cast(uint2, read_vt(src));
        const uint2 a1 = __builtin_bit_cast(uint2, read_vt(src + 16 * 128));
        return make_uint4(a0.x, a0.y, a1.x, a1.y);
      };
      uint4 vr[R];
#pragma unroll
      for (int i = 0; i < R; ++i) vr[i] = vread(i);
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, vr[dt % R]);
        if (dt + R < DV / 16) vr[dt % R] = vread(dt + R);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      auto vread = [&](int dt) -> uint2 { return lds_tr8(tile + vt[dt & 3] + (dt >> 2) * F8_GS); };
      uint2 vr[R];
#pragma unroll
      for (int i = 0; i < R; ++i) vr[i] = vread(i);
      bf16x8_t a = __builtin_bit_cast(bf16x8_t, fp8x8_to_bf16x8(vr[0].x, vr[0].y));
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) {
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[dt], 0, 0, 0);
        if (dt + R < DV / 16) vr[dt % R] = vread(dt + R);
        if (dt + 1 < DV / 16)
          a = __builtin_bit_cast(bf16x8_t, fp8x8_to_bf16x8(vr[(dt + 1) % R].x, vr[(dt + 1) % R].y));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // One 32-key step. The fast variant never touches the accumulators with
  // VALU code and returns false (before consuming the step) if a row's max
  // jumped more than BIG_SLACK above its reference; the slow variant rescales.
  auto compute = [&](const char* tile, int ts, auto slow_tag) -> bool {
    constexpr bool SLOW = decltype(slow_tag)::value;
    f32x4_t sacc[2];
    qk(tile, sacc);
    float x[2][4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[mi][e] = sacc[mi][e];
    // a step that reaches a row's limit, or whose page id was out of range
    if (tile_bad || __builtin_amdgcn_ballot_w64(ts + 32 > limit)) {
      // bf16: the lane group read afresh, which shortens the tile loop's
      // schedule (3% at 64 x 128 heads, 1-2k keys); for fp8 the same change
      // lengthens it (2% at 32 x 4 x 128 rows, 0.5-16k keys), so fp8 keeps
      // the value held from the prologue
      const int gk = 4 * (F8 ? g : fresh_lane() >> 4);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = ts + 16 * mi + gk + e;
          x[mi][e] = key < limit && !tile_bad ? x[mi][e] : -INFINITY;
        }
    }
    float tmax = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
    tmax = max4_groups(tmax) * scale_row;
    if constexpr (!SLOW) {
      if (m_run == -INFINITY) m_run = tmax;   // o and l of this row are still zero
      if (__builtin_amdgcn_ballot_w64(tmax > m_run + BIG_SLACK)) return false;
    } else {
      const bool need = tmax > m_run;
      if (__builtin_amdgcn_ballot_w64(need)) {
        float alpha = 1.f;
        if (need) {
          alpha = exp2f(m_run - tmax);   // m_run = -inf gives 0
          m_run = tmax;
        }
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < DV / 16; ++d) o[d] *= alpha;
      }
    }
    // a row without any key so far keeps m = -inf: a finite stand-in makes its
    // masked scores (-inf) give exp2(-inf) = 0, never NaN
    const float neg_m = -fmaxf(m_run, -1e30f);
    float e[2][4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        e[mi][jj] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[mi][jj], scale_row, neg_m));
        l_run += e[mi][jj];
      }
    const bf16x8_t pb = __builtin_bit_cast(
        bf16x8_t, make_uint4(pack_bf16x2(e[0][0], e[0][1]), pack_bf16x2(e[0][2], e[0][3]),
                             pack_bf16x2(e[1][0], e[1][1]), pack_bf16x2(e[1][2], e[1][3])));
    pv(tile, pb);
    return true;
  };

  // Make slot j resident for every wave: wait for this wave's transfers of
  // it (three slots are in flight at most), zero the keys past the end in
  // this wave's transfers, barrier, then issue slot j + 3 into the slot every
  // wave finished with before the barrier.
  auto prepare = [&](int j) -> const char* {
    char* cur = smem + (j & 3) * Y_SLOT;
    if (dma_wave) {
      mem_fence_compiler();
      const int ahead = min(2, ntiles - 1 - j);
      if (ahead >= 2)
        wait_vmcnt<2 * Y_NDMA>();
      else if (ahead == 1)
        wait_vmcnt<Y_NDMA>();
      else
        wait_vmcnt<0>();
      mem_fence_compiler();
    }
    const int nv = valid_keys(j);
    tile_bad = nv < 0;
    bad_page |= tile_bad;
    if (dma_wave && nv < KT) {
#pragma unroll
      for (int i = 0; i < Y_NDMA; ++i) {
        const int n = Y_NDMA * w + i;
        const int key = F8 ? 32 * (n >= 18) + 16 * ((n - 18 * (n >= 18)) & 1) + (lane >> 2)
                           : 8 * (n & 3) + (lane >> 3);
        if (key >= nv) *reinterpret_cast<uint4*>(cur + n * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
      }
    }
    __syncthreads();
    if (dma_wave && j + 3 < ntiles) issue(j + 3);
    return cur;
  };

  // tile of the sub-step u (fp8: two 32-key steps per slot)
  auto step_tile = [&](const char* cur, int u) -> const char* { return F8 ? cur + u * F8_TILE : cur; };
  constexpr int SUB = F8 ? 2 : 1;
  int j = 0, u = 0;
  const char* cur = nullptr;
  bool jumped = false;
  for (; j < ntiles; ++j) {
    cur = prepare(j);
    if (!wave_active) continue;
    for (u = 0; u < SUB; ++u) {
      const int ts = t0 + KT * j + 32 * u;
      if (ts >= t1) break;
      if (!compute(step_tile(cur, u), ts, std::false_type{})) {
        jumped = true;
        break;
      }
    }
    if (jumped) break;
  }
  if (jumped) {   // rare: finish with rescaling, from sub-step u of the resident slot j
    for (; u < SUB; ++u) {
      const int ts = t0 + KT * j + 32 * u;
      if (ts < t1) compute(step_tile(cur, u), ts, std::true_type{});
    }
    for (++j; j < ntiles; ++j) {
      cur = prepare(j);
      for (u = 0; u < SUB; ++u) {
        const int ts = t0 + KT * j + 32 * u;
        if (ts < t1) compute(step_tile(cur, u), ts, std::true_type{});
      }
    }
  }

  flag_bad_page(p.flags, bad_page);

  // ---- write this wave's rows: final (slot < 0) or split partial ----
  const float l_row = wave_sum_across_groups(l_run);
  const bool empty = !(l_row > 0.f);
  const float inv = empty ? 0.f : p.out_scale / l_row;
  int kexp = 0;   // split partials: fp16 o * 2^k (partial_exponent)
  if (slot >= 0) {
    float amax = 0.f;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(o[dt][e]));
    kexp = min(partial_exponent(wave_max_across_groups(amax) * inv), 127 - __builtin_amdgcn_frexp_expf(inv));
  }
  // The wave's 16 rows leave in 8 groups of 64 dims; each store covers 8
  // whole rows of a group (whole_row_runs), so every lane takes part in the
  // exchange and a store goes out only for a row of the sequence. Lane
  // values are derived afresh here, so that nothing computed for the
  // epilogue is held (and spilled) across the tile loop.
  const float fs = __builtin_ldexpf(inv, kexp);
  const int ln_e = fresh_lane(), c16e = ln_e & 15, ge = ln_e >> 4;
  const int r_lo = 16 * w + (c16e & 7), r_hi = r_lo + 8;   // item rows of the two stores
  const bool ok_lo = rg * Y_RGS + r_lo < p.rows, ok_hi = rg * Y_RGS + r_hi < p.rows;
  char* dst_lo;
  char* dst_hi;
  if (slot < 0) {
    const size_t orow0 = (size_t)b * p.rows + rg * Y_RGS;
    dst_lo = reinterpret_cast<char*>(p.out + (orow0 + r_lo) * DV);
    dst_hi = reinterpret_cast<char*>(p.out + (orow0 + r_hi) * DV);
  } else {
    dst_lo = reinterpret_cast<char*>(p.part_o + ((size_t)slot * Y_RGS + r_lo) * DV);
    dst_hi = reinterpret_cast<char*>(p.part_o + ((size_t)slot * Y_RGS + r_hi) * DV);
  }
  const int col = whole_row_col(c16e, ge);
#pragma unroll
  for (int k = 0; k < DV / 64; ++k) {
    uint32_t pk[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4_t v = o[4 * k + i] * fs;
      if (slot < 0) {
        pk[i][0] = pack_bf16x2(v[0], v[1]);
        pk[i][1] = pack_bf16x2(v[2], v[3]);
      } else {
        const uint2 h = __builtin_bit_cast(uint2, __builtin_convertvector(v, f16x4_t));
        pk[i][0] = h.x;
        pk[i][1] = h.y;
      }
    }
    uint4 lo, hi;
    whole_row_runs(pk, c16e, lo, hi);
    if (ok_lo) *reinterpret_cast<uint4*>(dst_lo + 128 * k + col) = lo;
    if (ok_hi) *reinterpret_cast<uint4*>(dst_hi + 128 * k + col) = hi;
  }
  const int row_e = rg * Y_RGS + 16 * w + c16e;   // this lane's own row
  if (row_e < p.rows && ge == 0) {
    const float lse2 = empty ? -INFINITY : m_run + log2f(l_row);
    if (slot < 0) {
      if (p.lse != nullptr) p.lse[(size_t)b * p.rows + row_e] = lse2 * LN2;
    } else {
      p.part_lse[(size_t)slot * Y_RGS + 16 * w + c16e] = lse2;
      p.part_scale[(size_t)slot * Y_RGS + 16 * w + c16e] = kexp;
    }
  }
}

}  // namespace

namespace mla_detail {

void launch_wide128(int kv_dtype, dim3 grid, hipStream_t st, const FwdParams& fp) {
  if (kv_dtype == MLA_DTYPE_BF16)
    hipLaunchKernelGGL((mla_decode_wide128<MLA_DTYPE_BF16>), grid, dim3(Y_THREADS), 0, st, fp);
  else
    hipLaunchKernelGGL((mla_decode_wide128<MLA_DTYPE_FP8_E4M3FN>), grid, dim3(Y_THREADS), 0, st, fp);
}

}  // namespace mla_detail
