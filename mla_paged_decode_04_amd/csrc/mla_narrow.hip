// Paged MLA decode, <= 16 query rows per sequence (the HBM-bound regime of
// the 16-head cases): decode attention of MLA in its MQA form ("[WIP][Attention]
// FlashAttn MLA", description) over a paged bf16 or fp8 e4m3fn cache
// ("[Attention] Blackwell FP8 MLA support with CUTLASS_MLA backend", review
// thread: the kernel test's parameters).
#include <type_traits>

#include "mla_internal.h"

using namespace mla_detail;

namespace {

// Final step of a work item. Each of the 4 waves holds, for the 16 rows of its
// row tile (one row per lane, lane groups splitting the dims), the running max
// m (base 2), its share of the running sum, and unnormalised O^T. The KS
// waves that share a row tile are merged through LDS (weights 2^(m_k - M)),
// then the rows are written as final bf16 out + natural-log lse (slot < 0), or
// as a split partial (fp16 normalised o * 2^k and base-2 lse). Every wave must be
// done with `smem` before the call.
template <int KS>
__device__ __forceinline__ void merge_and_store(const FwdParams& p, char* smem,
                                                const f32x4_t (&o)[DV / 16], float m_run,
                                                float l_run, int b, int rg, int slot) {
  constexpr int RGS = 16 * (4 / KS);
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const float l_row = wave_sum_across_groups(l_run);
  float* ost = reinterpret_cast<float*>(smem);                        // [4][16][OSTRIDE]
  float* mls = reinterpret_cast<float*>(smem + 4 * 16 * OSTRIDE * 4);  // [4][16][2]
  {
    float* dst = ost + (w * 16 + c16) * OSTRIDE + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt)
      *reinterpret_cast<f32x4_t*>(dst + 16 * dt) = o[dt];
    if (g == 0) {
      mls[(w * 16 + c16) * 2] = m_run;
      mls[(w * 16 + c16) * 2 + 1] = l_row;
    }
  }
  __syncthreads();

  // 16 threads per row; thread c of row rr handles dims 4c + 64i (i = 0..7):
  // every LDS read and global write of 16 threads is one contiguous run
  static_assert(KS == 4 && RGS == 16, "one 16-row tile merged over four waves");
  const int rr = tid >> 4;
  const int c4 = (tid & 15) * 4;
  float mk[KS], wk[KS];
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    mk[k] = mls[(k * 16 + rr) * 2];
    M = fmaxf(M, mk[k]);
  }
  float lsum = 0.f;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    wk[k] = mk[k] == -INFINITY ? 0.f : exp2f(mk[k] - M);
    lsum += wk[k] * mls[(k * 16 + rr) * 2 + 1];
  }
  const int grow = rg * RGS + rr;
  const bool row_ok = grow < p.rows;
  const bool empty = !(lsum > 0.f);
  const float inv = empty ? 0.f : p.out_scale / lsum;
  const float lse2 = empty ? -INFINITY : M + log2f(lsum);
  const size_t orow = (size_t)b * p.rows + grow;
  if (!row_ok) return;
  f32x4_t acc[DV / 64];
#pragma unroll
  for (int i = 0; i < DV / 64; ++i) {
    f32x4_t a = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k)
      a += wk[k] * *reinterpret_cast<const f32x4_t*>(ost + (k * 16 + rr) * OSTRIDE + c4 + 64 * i);
    acc[i] = a * inv;
  }
  if (slot < 0) {
    uint16_t* dst = p.out + orow * DV + c4;
#pragma unroll
    for (int i = 0; i < DV / 64; ++i)
      *reinterpret_cast<uint2*>(dst + 64 * i) =
          make_uint2(pack_bf16x2(acc[i][0], acc[i][1]), pack_bf16x2(acc[i][2], acc[i][3]));
    if (p.lse != nullptr && c4 == 0) p.lse[orow] = lse2 * LN2;
  } else {
    // fp16 o * 2^k (partial_exponent); the row's 512 dims are spread over 16
    // consecutive lanes
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < DV / 64; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(acc[i][e]));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const int kexp = partial_exponent(amax);
    _Float16* dst = p.part_o + ((size_t)slot * RGS + rr) * DV + c4;
#pragma unroll
    for (int i = 0; i < DV / 64; ++i) {
      const f32x4_t sv = f32x4_t{__builtin_ldexpf(acc[i][0], kexp), __builtin_ldexpf(acc[i][1], kexp),
                                 __builtin_ldexpf(acc[i][2], kexp), __builtin_ldexpf(acc[i][3], kexp)};
      *reinterpret_cast<f16x4_t*>(dst + 64 * i) = __builtin_convertvector(sv, f16x4_t);
    }
    if (c4 == 0) {
      p.part_lse[(size_t)slot * RGS + rr] = lse2;
      p.part_scale[(size_t)slot * RGS + rr] = kexp;
    }
  }
}

// ---------------------------------------------------------------------------
// decode kernel for <= 16 query rows per sequence (HBM-bound regime)
// ---------------------------------------------------------------------------
//
// Every wave streams its own 16-key tiles (keys t0 + 16*j for j = w, w+4, ...)
// straight from HBM into a private double buffer in LDS with
// global_load_lds_dwordx4 (no staging registers, no workgroup barrier per
// tile): while it computes tile j, tile j+4 is in flight. Tile layout in LDS:
// [9 column groups of 128 B][16 keys][8 x 16-byte chunks], chunk position
// XOR-swizzled by key & 7; the DMA lanes pick their global chunk so the LDS
// side is always 64 consecutive 16-byte slots. bf16 caches run S^T and O^T on
// bf16 MFMAs; fp8 caches (32-key tiles) run S^T on the fp8 MFMA with q split
// into exact e4m3fn hi/lo codes, and convert only the V operand to bf16.

constexpr int H16_KT = 16;                      // keys per wave tile
constexpr int H16_TILE = H16_KT * D * 2;        // 18432 bytes (bf16)
constexpr int H16_DMA = H16_TILE / 1024;        // 18 wave-wide 1 KB transfers
constexpr int H16_GSTRIDE = H16_KT * 128;       // bytes per 128-byte column group

// fp8 tiles: 32 keys x 576 bytes = 18432 bytes, laid out as
// [9 column groups of 64 B][32 keys][4 x 16-byte chunks] with the chunk
// position XOR-swizzled by f(key) = key bit 2 + 2 * key bit 4. With it the
// 16-byte K reads and the 8-byte transposed V reads below are free of LDS
// bank conflicts (measured on MI355X with the bank-conflict counter on each
// access pattern alone; the swizzle ((key >> 2) + (key >> 4)) & 3 doubled the
// LDS cycles of both).
constexpr int F8_KT = 32;
constexpr int F8_GSTRIDE = F8_KT * 64;

__device__ __forceinline__ int f8_swz(int key) { return ((key >> 2) & 1) | (((key >> 4) & 1) << 1); }

// 8 e4m3fn codes -> 8 bf16 (exact).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8_v(uint2 w) {
  return __builtin_bit_cast(bf16x8_t, fp8x8_to_bf16x8(w.x, w.y));
}

__device__ __forceinline__ uint2 read_vt8(const char* p) {
  typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(p)));
}

template <int KVT>
__global__ __launch_bounds__(NTHREADS, 1) void mla_decode_narrow(FwdParams p) {
  constexpr bool F8 = KVT == MLA_DTYPE_FP8_E4M3FN;
  constexpr int KT = F8 ? F8_KT : H16_KT;          // keys per wave tile
  constexpr int ROWB = F8 ? D : D * 2;             // bytes per cached row
  constexpr int TILE = KT * ROWB;                  // 18432 either way
  constexpr int NDMA = TILE / 1024;                // 18
  static_assert(TILE == H16_TILE, "same LDS budget for both caches");
  __shared__ __attribute__((aligned(1024))) char smem[4 * 2 * H16_TILE];   // 147456 bytes

  // The item count and this workgroup's item are read in one memory round
  // trip: the grid never exceeds the item array's capacity (rounded up to 8
  // items, within its 256-byte-aligned region), so the item read is in bounds
  // even for a workgroup that then finds it has no item.
  const int item_id = blockIdx.x;
  const int32_t* it = p.items + (size_t)item_id * ITEM_INTS;
  const int n_items = min(p.header[0], p.max_items);
  // work-item fields are uniform: keep them (and all tile addressing derived
  // from them) in SGPRs, so no vector load ever enters the DMA vmcnt queue
  const int b = __builtin_amdgcn_readfirstlane(it[0]);
  const int t0 = __builtin_amdgcn_readfirstlane(it[2]);
  const int t1 = __builtin_amdgcn_readfirstlane(it[3]);
  const int slot = __builtin_amdgcn_readfirstlane(it[4]);
  // (the asm pins the loads, and the launch fields the first block-table read
  // needs, ahead of the branch)
  asm volatile("" ::"s"(n_items), "s"(b), "s"(t0), "s"(t1), "s"(slot), "s"(p.bs), "s"(p.max_blocks),
               "s"(p.block_table), "s"(p.seq_lens));
  if (item_id >= n_items) return;
  if (!item_in_range(p, 16, b, 0, t0, t1, slot)) {
    flag_bad_item(p.flags);
    return;
  }

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c16 = lane & 15;

  // The block table and seq_lens are read-only for the whole kernel: reading
  // them through the constant address space keeps these uniform loads on the
  // scalar unit, so they never enter the vmcnt queue the DMA waits below count
  // on. The length is requested here and used only after the first tile was
  // issued, so its load shares a round trip with the first block-table read.
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const int L_raw = ((const_i32*)p.seq_lens)[b];
  const int row = c16;
  const bool row_ok = row < p.rows;
  int limit = 0;   // keys this row sees, set once the first tile is in flight

  // q operands, loaded below (bf16: after this wave's first tile was
  // requested; fp8: staged in LDS ahead of it). bf16 caches: qb[s] holds dims
  // 32s + 8g .. +7 of row c16 (16x16x32 bf16 MFMA). fp8 caches: S^T runs on the 16x16x128 f8f6f4 MFMA with both
  // operands e4m3fn: the keys' codes as stored, and the row q * 2^qe split
  // into hi + lo codes; q8h/q8l[s] hold dims 128s + 32g .. +31, q8r holds
  // rope dims 32(g & 1) .. +31 as hi codes (g < 2) or lo codes (g >= 2), so
  // one MFMA takes both halves of the 64 rope dims.
  constexpr int QB = F8 ? 1 : D / 32;
  bf16x8_t qb[QB];
  i32x8_t q8h[4], q8l[4], q8r;
  float scale_row = p.scale_log2;   // fp8: times 2^-qe

  f32x4_t o[DV / 16];
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  // ---- lane constants (LDS byte offsets inside a tile, DMA source offsets) ----
  uint32_t dma_lane[2];
  int kb[2][2];   // K operand: bf16 [M tile][s & 1], add (s >> 1) * column-group stride;
                  // fp8 [M tile][chunk h], add the column-group offset
  int vt[4];      // V^T operand: [dt & 3], add (dt >> 2) * column-group stride
  if constexpr (!F8) {
    dma_lane[0] = dma_lane[1] = (lane >> 3) * ROWB + (((lane & 7) ^ (lane >> 3)) << 4);
    kb[0][0] = c16 * 128 + ((g ^ (c16 & 7)) << 4);
    kb[0][1] = c16 * 128 + (((4 + g) ^ (c16 & 7)) << 4);
    kb[1][0] = kb[0][0];
    kb[1][1] = kb[0][1];
    const int j = c16 >> 2, q = c16 & 3;
    const int lanex = (q >> 1) ^ ((g & 1) << 2) ^ j;
#pragma unroll
    for (int c = 0; c < 4; ++c) vt[c] = (4 * g + j) * 128 + (((2 * c) ^ lanex) << 4) + (q & 1) * 8;
  } else {
    // DMA transfer n: column group n >> 1, keys 16*(n & 1) + (lane >> 2), chunk
    // position lane & 3; f(key) = ((lane >> 4) & 1) + 2 (n & 1).
#pragma unroll
    for (int h = 0; h < 2; ++h)
      dma_lane[h] = (lane >> 2) * ROWB + (((lane & 3) ^ (((lane >> 4) & 1) | (2 * h))) << 4);
    // K: key 16*mi + c16, bytes 32*g .. +31 of a 128-byte step -> column
    // group 2*step + (g >> 1), chunks 2*(g & 1) + h (h = 0, 1); the rope step
    // reads column group 8 from every g. The 16 lanes of one quarter-wave hit
    // 16 different 16-byte bank groups.
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        kb[mi][h] = (16 * mi + c16) * 64 + (((2 * (g & 1) + h) ^ f8_swz(16 * mi + c16)) << 4);
    // V^T: lane s = 2*jj + q supplies V[key_jj][16*dt + 8*q ..+7] with key_jj =
    // 4g + jj (jj < 4) or 16 + 4g + jj - 4, so ds_read_b64_tr_b8 hands lane
    // c16 the 8 values V[key_0..7][16*dt + c16].
    const int jj = c16 >> 1, q = c16 & 1;
    const int key = jj < 4 ? 4 * g + jj : 16 + 4 * g + (jj - 4);
#pragma unroll
    for (int c = 0; c < 4; ++c) vt[c] = key * 64 + ((c ^ f8_swz(key)) << 4) + q * 8;
  }
  constexpr int GSTRIDE = F8 ? F8_GSTRIDE : H16_GSTRIDE;

  const_i32* bt = (const_i32*)(p.block_table + (size_t)b * p.max_blocks);
  // the block size is 64 or 128 (checked on the host): page and row offset
  // are a shift and a mask
  const int bsh = p.bs == 128 ? 7 : 6;
  char* wbuf = smem + w * 2 * H16_TILE;
  const int ntiles = (t1 - t0 + KT - 1) / KT;

  // Issue the NDMA transfers of tile j into dst (always NDMA VMEM
  // instructions, so the vmcnt arithmetic below is exact). Keys past the end
  // are fetched from a valid row of the page and zeroed after arrival.
  auto issue = [&](int j, char* dst) {
    const int ts = t0 + KT * j;
    int page = bt[ts >> bsh];
    if (page < 0 || page >= p.num_blocks) page = 0;
    const char* src = reinterpret_cast<const char*>(p.kv) + ((size_t)page * p.bs + (ts & (p.bs - 1))) * ROWB;
    const uint32_t l0 = lds_addr(dst);
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
      if constexpr (!F8)
        lds_dma16_nt(src + (n & 1) * 8 * ROWB + (n >> 1) * 128, dma_lane[0], l0 + n * 1024);
      else
        lds_dma16(src + (n & 1) * 16 * ROWB + (n >> 1) * 64, dma_lane[n & 1], l0 + n * 1024);
    }
  };
  // keys of tile j that hold data; -1 when its page id is out of range (the
  // tile is then zeroed and every key masked)
  auto valid_keys = [&](int j) {
    const int ts = t0 + KT * j;
    int page = bt[ts >> bsh];
    if (page < 0 || page >= p.num_blocks) return -1;
    return min(KT, t1 - ts);
  };
  bool bad_page = false;
  bool tile_ok = true;
  auto fix_tail = [&](int nv, char* buf) {
    if (nv >= KT) return;
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
      const int key = F8 ? (n & 1) * 16 + (lane >> 2) : (n & 1) * 8 + (lane >> 3);
      if (key >= nv) *reinterpret_cast<uint4*>(buf + n * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
    }
  };

  // Make tile j (this wave's itn-th) resident: issue the DMA of tile j + 4,
  // wait for tile j, zero its keys past the end. Returns its LDS buffer.
  auto prepare = [&](int j, int itn) -> const char* {
    char* cur = wbuf + (itn & 1) * H16_TILE;
    const bool has_next = j + 4 < ntiles;
    mem_fence_compiler();
    if (has_next) {
      issue(j + 4, wbuf + ((itn + 1) & 1) * H16_TILE);
      wait_vmcnt<NDMA>();
    } else {
      wait_vmcnt<0>();
    }
    mem_fence_compiler();
    const int nv = valid_keys(j);
    tile_ok = nv >= 0;
    bad_page |= !tile_ok;
    fix_tail(nv, cur);
    return cur;
  };

  // One tile: S^T, softmax, O^T += V^T P^T. The fast variant never touches
  // the accumulators with VALU code and returns false (before consuming the
  // tile) if a row's max jumped more than BIG_SLACK above its reference.
  auto compute = [&](const char* cur, int ts, auto slow_tag) -> bool {
    constexpr bool SLOW = decltype(slow_tag)::value;
    constexpr int MT = KT / 16;
    f32x4_t sacc[MT];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) sacc[mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (!F8) {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(cur + kb[mi][s & 1] + (s >> 1) * GSTRIDE);
          sacc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[s], sacc[mi], 0, 0, 0);
        }
      }
    } else {
      // 32 consecutive key bytes per lane: two 16-byte chunks of one key row
      auto k8 = [&](const char* base, int mi) {
        const uint4 x = *reinterpret_cast<const uint4*>(base + kb[mi][0]);
        const uint4 y = *reinterpret_cast<const uint4*>(base + kb[mi][1]);
        return i32x8_t{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
      };
      const char* kg = cur + (g >> 1) * GSTRIDE;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        i32x8_t a[MT];
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) a[mi] = k8(kg + 2 * s * GSTRIDE, mi);
        // hi of both M tiles, then lo: no MFMA waits on the one before it
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
          sacc[mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[mi], q8h[s], sacc[mi], 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
          sacc[mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[mi], q8l[s], sacc[mi], 0, 0, 0, 0, 0, 0);
      }
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
        sacc[mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k8(cur + 8 * GSTRIDE, mi), q8r, sacc[mi], 0, 0,
                                                                    0, 0, 0, 0);
    }

    float x[MT][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int key = ts + 16 * mi + 4 * g + jj;
        float v = sacc[mi][jj] * scale_row;
        v = key < limit && tile_ok ? v : -INFINITY;
        x[mi][jj] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = wave_max_across_groups(tmax);
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
    float pv[MT][4];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float e = m_run == -INFINITY ? 0.f : exp2f(x[mi][jj] - m_run);
        pv[mi][jj] = e;
        l_run += e;
      }

    if constexpr (!F8) {
      const s16x4_t pb = __builtin_bit_cast(
          s16x4_t, make_uint2(pack_bf16x2(pv[0][0], pv[0][1]), pack_bf16x2(pv[0][2], pv[0][3])));
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) {
        const s16x4_t a = read_vt(cur + vt[dt & 3] + (dt >> 2) * GSTRIDE);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[dt], 0, 0, 0);
      }
    } else {
      // k-slots 0..3: keys 4g..4g+3 of M tile 0; 4..7: of M tile 1 (same in A)
      const bf16x8_t pb = __builtin_bit_cast(
          bf16x8_t, make_uint4(pack_bf16x2(pv[0][0], pv[0][1]), pack_bf16x2(pv[0][2], pv[0][3]),
                               pack_bf16x2(pv[1][0], pv[1][1]), pack_bf16x2(pv[1][2], pv[1][3])));
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) {
        const bf16x8_t a = fp8x8_to_bf16x8_v(read_vt8(cur + vt[dt & 3] + (dt >> 2) * GSTRIDE));
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[dt], 0, 0, 0);
      }
    }
    return true;
  };

  int j = w, itn = 0;
  const char* cur = nullptr;
  if constexpr (F8) {
    // q reaches LDS by DMA, into this wave's second tile buffer (free until
    // tile j + 4 is requested), ahead of tile 0: the wait for it below leaves
    // tile 0 in flight, and the split into e4m3fn codes overlaps that. Layout
    // [18 blocks of 32 dims][16 rows][64 bytes]; rows past the end read the
    // last valid row (their values are replaced by zeros below).
    const int qr = min(lane >> 2, p.rows - 1);
    const char* qsrc = uniform_ptr(reinterpret_cast<const char*>(p.q + (size_t)b * p.rows * D));
    const uint32_t ql = lds_addr(wbuf + H16_TILE);
    const uint32_t qoff = qr * (D * 2) + (lane & 3) * 16;
#pragma unroll
    for (int n = 0; n < NDMA; ++n) lds_dma16(qsrc + n * 64, qoff, ql + n * 1024);
  }
  if (w < ntiles) issue(w, wbuf);
  const int L = min(max(L_raw, 0), p.max_keys);
  if (row_ok) {
    const int tok = row / p.heads;
    const int vis = p.causal ? L - p.s_q + 1 + tok : L;
    limit = min(vis, t1);
  }
  // bf16: q is loaded while the first tile is in flight. Its loads are
  // consumed here, so the compiler's own vmcnt wait for them (which also
  // covers the older tile transfers) sits before the tile loop, not inside it
  // (it cannot see the DMAs).
  if constexpr (!F8) {
    const uint16_t* qrow = p.q + ((size_t)b * p.rows + (row_ok ? row : 0)) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      qb[s] = __builtin_bit_cast(bf16x8_t, load16_masked(qrow + 32 * s + 8 * g, row_ok));
    }
#pragma unroll
    for (int s = 0; s < D / 32; ++s) asm volatile("" ::"v"(qb[s]));
  } else {
    // q's transfers are the oldest: with tile 0's NDMA behind them in flight
    mem_fence_compiler();
    if (w < ntiles)
      wait_vmcnt<NDMA>();
    else
      wait_vmcnt<0>();
    mem_fence_compiler();
    const char* qs = wbuf + H16_TILE;
    // dims 128s + 32g + 8c (s < 4) and rope dims 512 + 32(g & 1) + 8c (s = 4):
    // 32-dim block 4s + g (or 16 + (g & 1)), 16-byte chunk c of row c16
    uint4 v[5][4];
    float qmax = 0.f;
#pragma unroll
    for (int s = 0; s < 5; ++s)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int blk = s < 4 ? 4 * s + g : 16 + (g & 1);
        v[s][c] = load16_masked(qs + blk * 1024 + c16 * 64 + c * 16, row_ok);
        const uint32_t w4[4] = {v[s][c].x, v[s][c].y, v[s][c].z, v[s][c].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          qmax = fmaxf(qmax, fmaxf(fabsf(__builtin_bit_cast(float, w4[i] << 16)),
                                   fabsf(__builtin_bit_cast(float, w4[i] & 0xFFFF0000u))));
      }
    // row scale 2^qe puts the row's largest |q| in [128, 256); scores are then
    // sums of products of exact e4m3fn values, and 2^-qe joins the score scale
    qmax = wave_max_across_groups(qmax);
    const int qe = qmax > 0.f && qmax < INFINITY ? 8 - __builtin_amdgcn_frexp_expf(qmax) : 0;
    const float qmul = __builtin_ldexpf(1.f, qe);
    scale_row = p.scale_log2 * __builtin_ldexpf(1.f, -qe);
#pragma unroll
    for (int s = 0; s < 5; ++s) {
      uint32_t h8[8], l8[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) split_fp8x8(v[s][c], qmul, h8 + 2 * c, l8 + 2 * c);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (s < 4) {
          q8h[s < 4 ? s : 0][i] = static_cast<int>(h8[i]);
          q8l[s < 4 ? s : 0][i] = static_cast<int>(l8[i]);
        } else {
          q8r[i] = static_cast<int>(g < 2 ? h8[i] : l8[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // per dword: a 256-bit operand would be an x86 register class in the host pass
#pragma unroll
      for (int s = 0; s < 4; ++s) asm volatile("" ::"v"(q8h[s][i]), "v"(q8l[s][i]));
      asm volatile("" ::"v"(q8r[i]));
    }
  }
  for (; j < ntiles; j += 4, ++itn) {
    cur = prepare(j, itn);
    if (!compute(cur, t0 + KT * j, std::false_type{})) break;
  }
  if (j < ntiles) {   // rare: finish with rescaling, starting at the resident tile j
    compute(cur, t0 + KT * j, std::true_type{});
    for (j += 4, ++itn; j < ntiles; j += 4, ++itn)
      compute(prepare(j, itn), t0 + KT * j, std::true_type{});
  }
  flag_bad_page(p.flags, bad_page);
  __syncthreads();
  merge_and_store<4>(p, smem, o, m_run, l_run, b, 0, slot);
}

}  // namespace

namespace mla_detail {

void launch_narrow(int kv_dtype, dim3 grid, hipStream_t st, const FwdParams& fp) {
  if (kv_dtype == MLA_DTYPE_BF16)
    hipLaunchKernelGGL((mla_decode_narrow<MLA_DTYPE_BF16>), grid, dim3(NTHREADS), 0, st, fp);
  else
    hipLaunchKernelGGL((mla_decode_narrow<MLA_DTYPE_FP8_E4M3FN>), grid, dim3(NTHREADS), 0, st, fp);
}

}  // namespace mla_detail
