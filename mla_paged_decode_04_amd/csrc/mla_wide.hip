// Paged MLA decode, > 16 query rows per sequence (the MFMA-heavy regime of
// the 128-head cases).
#include <type_traits>

#include "mla_internal.h"

using namespace mla_detail;

namespace {

// ---------------------------------------------------------------------------
// decode kernel for up to 64 query rows per item (MFMA-heavy regime)
// ---------------------------------------------------------------------------
//
// The 4 waves share 32-key tiles streamed HBM -> LDS through a 4-deep ring,
// so three tiles are in flight while one is computed; one workgroup barrier
// per tile. Wave w owns 16 query rows. bf16 tiles are DMA'd straight into the
// bf16 layout [9 column groups of 128 B][32 keys][8 x 16 B], chunk position
// (c & 7) ^ (key & 7). fp8 tiles are DMA'd raw (row-major, 576 B per key) into
// a 4-deep ring and widened once per tile, by all 256 threads, into a
// double-buffered bf16 tile of the same layout, so every wave reads bf16.

constexpr int W_NTK = 32;                         // keys per tile
constexpr int W_TILE = W_NTK * D * 2;             // 36864 bytes (bf16 tile)
constexpr int W_RAW8 = W_NTK * D;                 // 18432 bytes (raw fp8 tile)
constexpr int W_GSTRIDE = W_NTK * 128;            // bytes per 128-byte column group
#ifndef QK_AHEAD
#define QK_AHEAD 8                                // K-operand LDS reads kept in flight
#endif

// Max over the four 16-lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48) with
// gfx950's row-swap permutes: v_permlane32_swap exchanges the two 32-lane
// halves of its operands, v_permlane16_swap the odd and even 16-lane rows
// (VALU only, no LDS round trip as with ds_bpermute). Issued from inline asm
// (not volatile, so it stays free to schedule): through the builtins the
// compiler folds max(swap result 0, swap result 1) to result 0. The s_nop
// pairs cover the VALU-write -> permlane hazards.
__device__ __forceinline__ float max_across_groups(float v) {
  float y = v;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(v), "+v"(y));
  v = fmaxf(v, y);
  y = v;
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(v), "+v"(y));
  return fmaxf(v, y);
}

__device__ __forceinline__ int w_off(int key, int c) {
  return (((c >> 3) * W_NTK + key) << 7) + (((c & 7) ^ (key & 7)) << 4);
}

template <int KVT, int RPW>
__global__ __launch_bounds__(NTHREADS, 1) void mla_decode_wide(FwdParams p) {
  static_assert(RPW == 1, "16 rows per wave");
  constexpr bool F8 = KVT == MLA_DTYPE_FP8_E4M3FN;
  constexpr int RGS = 4 * RPW * 16;                 // rows per work item
  constexpr int ROWB = F8 ? D : D * 2;              // bytes per cached row
  // bf16: ring of 4 tiles, 9 transfers per wave per tile.
  // fp8: ring of 4 raw tiles (waves 0-1 issue 9 transfers each) + 2 bf16 tiles.
  constexpr int NDMA = 9;
  __shared__ __attribute__((aligned(1024))) char smem[4 * W_TILE];   // 147456 bytes
  char* const raw8 = smem;                          // fp8: 4 x 18432
  char* const bfbuf = smem + (F8 ? 4 * W_RAW8 : 0); // fp8: 2 x 36864

  // XCD-aware item order: consecutive workgroups go to different XCDs, so
  // hand each XCD a contiguous run of items (the row groups and chunks of one
  // sequence then share that XCD's L2). The grid is a multiple of 8.
  const int n_items = min(p.header[0], p.max_items);
  const int per_xcd = (n_items + 7) >> 3;
  const int xw = blockIdx.x;
  if ((xw >> 3) >= per_xcd) return;
  const int item_id = (xw & 7) * per_xcd + (xw >> 3);
  if (item_id >= n_items) return;
  const int32_t* it = p.items + (size_t)item_id * ITEM_INTS;
  // uniform work-item fields, pinned to SGPRs (see the narrow kernel)
  const int b = __builtin_amdgcn_readfirstlane(it[0]);
  const int rg = __builtin_amdgcn_readfirstlane(it[1]);
  const int t0 = __builtin_amdgcn_readfirstlane(it[2]);
  const int t1 = __builtin_amdgcn_readfirstlane(it[3]);
  const int slot = __builtin_amdgcn_readfirstlane(it[4]);
  if (!item_in_range(p, RGS, b, rg, t0, t1, slot)) {
    flag_bad_item(p.flags);
    return;
  }

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int L = __builtin_amdgcn_readfirstlane(min(max(p.seq_lens[b], 0), p.max_keys));

  const int row_local = w * 16 + c16;
  const int row = rg * RGS + row_local;
  const bool row_ok = row < p.rows;
  int limit = 0;
  if (row_ok) {
    const int tok = row / p.heads;
    const int vis = p.causal ? L - p.s_q + 1 + tok : L;
    limit = min(vis, t1);
  }
  bf16x8_t qb[D / 32];
  {
    const uint16_t* qrow = p.q + ((size_t)b * p.rows + (row_ok ? row : 0)) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      qb[s] = __builtin_bit_cast(bf16x8_t, load16_masked(qrow + 32 * s + 8 * g, row_ok));
    }
  }
  // q loads complete here, before the first (compiler-invisible) DMA
#pragma unroll
  for (int s = 0; s < D / 32; ++s) asm volatile("" ::"v"(qb[s]));

  f32x4_t o[DV / 16];
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- lane constants ----
  // bf16 DMA: transfer n (0..35) = column group n >> 2, keys 8*(n & 3) + (lane >> 3)
  const uint32_t dma_lane = F8 ? lane * 16 : (lane >> 3) * ROWB + (((lane & 7) ^ (lane >> 3)) << 4);
  int kb[2][2];   // K operand [M tile][s & 1]; add (s >> 1) * W_GSTRIDE
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    kb[h][0] = (16 * h + c16) * 128 + ((g ^ (c16 & 7)) << 4);
    kb[h][1] = (16 * h + c16) * 128 + (((4 + g) ^ (c16 & 7)) << 4);
  }
  int vt[4];      // V^T operand [dt & 3]; add (dt >> 2) * W_GSTRIDE, second half + 16 rows
  {
    const int j = c16 >> 2, q = c16 & 3;
    const int lanex = (q >> 1) ^ ((g & 1) << 2) ^ j;
#pragma unroll
    for (int c = 0; c < 4; ++c) vt[c] = (4 * g + j) * 128 + (((2 * c) ^ lanex) << 4) + (q & 1) * 8;
  }

  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const_i32* bt = (const_i32*)(p.block_table + (size_t)b * p.max_blocks);
  // the block size is 64 or 128 (checked on the host): page and row offset
  // are a shift and a mask
  const int bsh = p.bs == 128 ? 7 : 6;
  const int ntiles = (t1 - t0 + W_NTK - 1) / W_NTK;
  // fp8 tiles are fetched by waves 0 and 1 only (18 transfers per tile)
  const bool dma_wave = !F8 || w < 2;

  // Issue this wave's NDMA transfers of tile j (exactly NDMA VMEM
  // instructions per participating wave; vmcnt arithmetic relies on it).
  auto issue = [&](int j) {
    const int ts = t0 + W_NTK * j;
    int page = bt[ts >> bsh];
    if (page < 0 || page >= p.num_blocks) page = 0;
    const char* src = reinterpret_cast<const char*>(p.kv) + ((size_t)page * p.bs + (ts & (p.bs - 1))) * ROWB;
    if constexpr (!F8) {
      const uint32_t l0 = lds_addr(smem + (j & 3) * W_TILE);
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int n = w * NDMA + i;
        lds_dma16_nt(src + (n & 3) * 8 * ROWB + (n >> 2) * 128, dma_lane, l0 + n * 1024);
      }
    } else {
      const uint32_t l0 = lds_addr(raw8 + (j & 3) * W_RAW8);
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int n = w * NDMA + i;
        lds_dma16_nt(src + n * 1024, dma_lane, l0 + n * 1024);
      }
    }
  };
  // keys of tile j that hold data; -1 when its page id is out of range (the
  // tile is then zeroed and every key masked)
  auto valid_keys = [&](int j) {
    const int ts = t0 + W_NTK * j;
    int page = bt[ts >> bsh];
    if (page < 0 || page >= p.num_blocks) return -1;
    return min(W_NTK, t1 - ts);
  };
  bool bad_page = false, tile_bad = false;
  // wait until this wave's transfers of tile j landed, given that tiles up to
  // j + ahead were issued after it
  auto wait_tile = [&](int ahead) {
    if (!dma_wave) return;
    if (ahead >= 2)
      wait_vmcnt<2 * NDMA>();
    else if (ahead == 1)
      wait_vmcnt<NDMA>();
    else
      wait_vmcnt<0>();
  };

  if (dma_wave) {
#pragma unroll
    for (int k = 0; k < 3; ++k)
      if (k < ntiles) issue(k);
  }

  // Make tile j resident for every wave (wait for this wave's transfers,
  // barrier, issue tile j + 3; fp8: widen to bf16). Returns the bf16 tile.
  auto prepare = [&](int j) -> const char* {
    mem_fence_compiler();
    wait_tile(min(2, ntiles - 1 - j));
    mem_fence_compiler();
    const int nv = valid_keys(j);
    tile_bad = nv < 0;
    bad_page |= tile_bad;
    const char* cur;
    if constexpr (!F8) {
      cur = smem + (j & 3) * W_TILE;
      if (nv < W_NTK) {   // zero this wave's slots of keys >= nv
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
          const int n = w * NDMA + i;
          const int key = (n & 3) * 8 + (lane >> 3);
          if (key >= nv)
            *reinterpret_cast<uint4*>(smem + (j & 3) * W_TILE + n * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
        }
      }
      __syncthreads();   // tile j complete; tile j-1 consumed by every wave
      if (dma_wave && j + 3 < ntiles) issue(j + 3);
    } else {
      __syncthreads();   // raw tile j landed; raw j-1 and bf16 tile (j-2) consumed
      if (dma_wave && j + 3 < ntiles) issue(j + 3);
      // widen raw tile j into bf16 tile j & 1: 1152 chunks of 16 codes
      char* dst = bfbuf + (j & 1) * W_TILE;
      const char* rsrc = raw8 + (j & 3) * W_RAW8;
#pragma unroll
      for (int i = 0; i < (W_RAW8 / 16 + NTHREADS - 1) / NTHREADS; ++i) {
        const int qc = i * NTHREADS + tid;
        if (qc < W_RAW8 / 16) {
          const int key = qc / (D / 16);
          const int c = 2 * (qc - key * (D / 16));
          uint4 v = *reinterpret_cast<const uint4*>(rsrc + qc * 16);
          uint4 lo = fp8x8_to_bf16x8(v.x, v.y), hi = fp8x8_to_bf16x8(v.z, v.w);
          if (key >= nv) lo = hi = make_uint4(0, 0, 0, 0);
          *reinterpret_cast<uint4*>(dst + w_off(key, c)) = lo;
          *reinterpret_cast<uint4*>(dst + w_off(key, c + 1)) = hi;
        }
      }
      __syncthreads();   // bf16 tile complete
      cur = dst;
    }
    return cur;
  };

  // One 32-key tile. The fast variant never touches the accumulators with
  // VALU code and returns false (before consuming the tile) if a row's max
  // jumped more than BIG_SLACK above its reference.
  auto compute = [&](const char* cur, int ts, auto slow_tag) -> bool {
    constexpr bool SLOW = decltype(slow_tag)::value;

    // ---- S^T for 32 keys (two M tiles) x this wave's 16 rows ----
    f32x4_t sacc[2];   // [M tile]: two independent accumulation chains
#pragma unroll
    for (int h = 0; h < 2; ++h) sacc[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(cur + kb[h][s & 1] + (s >> 1) * W_GSTRIDE);
        sacc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[s], sacc[h], 0, 0, 0);
      }
    }
    // Keep QK_AHEAD K-operand reads in flight ahead of the MFMAs: with one
    // wave per SIMD nothing else hides the LDS latency.
#pragma unroll
    for (int i = 0; i < QK_AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < D / 16 - QK_AHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < QK_AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);

    // ---- online softmax (lane = one row, 8 keys), on the raw scores: the
    // scale is folded into the max and into the exponent's FMA ----
    float x[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) x[h][jj] = sacc[h][jj];
    // a tile that reaches a row's limit, or whose page id was out of range
    if (tile_bad || __builtin_amdgcn_ballot_w64(ts + W_NTK > limit)) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int key = ts + 16 * h + 4 * g + jj;
          x[h][jj] = key < limit && !tile_bad ? x[h][jj] : -INFINITY;
        }
    }
    float tmax = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
    tmax = max_across_groups(tmax) * p.scale_log2;
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
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        e[h][jj] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[h][jj], p.scale_log2, neg_m));
        l_run += e[h][jj];
      }
    const bf16x8_t pb = __builtin_bit_cast(
        bf16x8_t, make_uint4(pack_bf16x2(e[0][0], e[0][1]), pack_bf16x2(e[0][2], e[0][3]),
                             pack_bf16x2(e[1][0], e[1][1]), pack_bf16x2(e[1][2], e[1][3])));

    // ---- O^T += V^T P^T over these 32 keys ----
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      const char* src = cur + vt[dt & 3] + (dt >> 2) * W_GSTRIDE;
      const s16x4_t a0 = read_vt(src);
      const s16x4_t a1 = read_vt(src + 16 * 128);
      const bf16x8_t a = __builtin_bit_cast(
          bf16x8_t, make_uint4(__builtin_bit_cast(uint2, a0).x, __builtin_bit_cast(uint2, a0).y,
                               __builtin_bit_cast(uint2, a1).x, __builtin_bit_cast(uint2, a1).y));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[dt], 0, 0, 0);
    }
      return true;
  };

  int j = 0;
  const char* cur = nullptr;
  for (; j < ntiles; ++j) {
    cur = prepare(j);
    if (!compute(cur, t0 + W_NTK * j, std::false_type{})) break;
  }
  if (j < ntiles) {   // rare: finish with rescaling, starting at the resident tile j
    compute(cur, t0 + W_NTK * j, std::true_type{});
    for (++j; j < ntiles; ++j) compute(prepare(j), t0 + W_NTK * j, std::true_type{});
  }

  flag_bad_page(p.flags, bad_page);

  // ---- write this wave's rows: final (slot < 0) or split partial ----
  const float l_row = wave_sum_across_groups(l_run);
  int kexp = 0;   // split partials: fp16 o * 2^k (partial_exponent)
  if (slot >= 0) {
    float amax = 0.f;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(o[dt][e]));
    const bool empty = !(l_row > 0.f);
    kexp = partial_exponent(wave_max_across_groups(amax) * (empty ? 0.f : p.out_scale / l_row));
  }
  // The wave's 16 rows leave in 8 groups of 64 dims; each store covers 8
  // whole rows of a group (whole_row_runs), so every lane takes part in the
  // exchange and a store goes out only for a row of the sequence.
  const bool empty = !(l_row > 0.f);
  const float inv = empty ? 0.f : p.out_scale / l_row;
  const int r_lo = 16 * w + (c16 & 7), r_hi = r_lo + 8;   // item rows of the two stores
  const bool ok_lo = rg * RGS + r_lo < p.rows, ok_hi = rg * RGS + r_hi < p.rows;
  char* dst_lo;
  char* dst_hi;
  if (slot < 0) {
    const size_t orow0 = (size_t)b * p.rows + rg * RGS;
    dst_lo = reinterpret_cast<char*>(p.out + (orow0 + r_lo) * DV);
    dst_hi = reinterpret_cast<char*>(p.out + (orow0 + r_hi) * DV);
  } else {
    dst_lo = reinterpret_cast<char*>(p.part_o + ((size_t)slot * RGS + r_lo) * DV);
    dst_hi = reinterpret_cast<char*>(p.part_o + ((size_t)slot * RGS + r_hi) * DV);
  }
  const int col = whole_row_col(c16, g);
#pragma unroll
  for (int k = 0; k < DV / 64; ++k) {
    uint32_t pk[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4_t v = o[4 * k + i] * inv;
      if (slot < 0) {
        pk[i][0] = pack_bf16x2(v[0], v[1]);
        pk[i][1] = pack_bf16x2(v[2], v[3]);
      } else {
        const f32x4_t sv = f32x4_t{__builtin_ldexpf(v[0], kexp), __builtin_ldexpf(v[1], kexp),
                                   __builtin_ldexpf(v[2], kexp), __builtin_ldexpf(v[3], kexp)};
        const uint2 h = __builtin_bit_cast(uint2, __builtin_convertvector(sv, f16x4_t));
        pk[i][0] = h.x;
        pk[i][1] = h.y;
      }
    }
    uint4 lo, hi;
    whole_row_runs(pk, c16, lo, hi);
    if (ok_lo) *reinterpret_cast<uint4*>(dst_lo + 128 * k + col) = lo;
    if (ok_hi) *reinterpret_cast<uint4*>(dst_hi + 128 * k + col) = hi;
  }
  if (row_ok && g == 0) {
    const float lse2 = empty ? -INFINITY : m_run + log2f(l_row);
    if (slot < 0) {
      if (p.lse != nullptr) p.lse[(size_t)b * p.rows + row] = lse2 * LN2;
    } else {
      p.part_lse[(size_t)slot * RGS + row_local] = lse2;
      p.part_scale[(size_t)slot * RGS + row_local] = kexp;
    }
  }
}

}  // namespace

namespace mla_detail {

void launch_wide(int kv_dtype, dim3 grid, hipStream_t st, const FwdParams& fp) {
  if (kv_dtype == MLA_DTYPE_BF16)
    hipLaunchKernelGGL((mla_decode_wide<MLA_DTYPE_BF16, 1>), grid, dim3(NTHREADS), 0, st, fp);
  else
    hipLaunchKernelGGL((mla_decode_wide<MLA_DTYPE_FP8_E4M3FN, 1>), grid, dim3(NTHREADS), 0, st, fp);
}

}  // namespace mla_detail
