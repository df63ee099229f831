// Paged MLA decode for MI355X (gfx950 / CDNA4): split planner, MFMA decode
// kernels and LSE combine, behind the C ABI declared in include/mla_decode.h.
//
// Operation: decode attention of MLA in its MQA form ("[WIP][Attention]
// FlashAttn MLA", description) with d = 576, dv = 512, one KV head, a paged
// cache in bf16 or fp8 e4m3fn ("[Attention] Blackwell FP8 MLA support with
// CUTLASS_MLA backend", review thread: the kernel test's parameters).
//
// Structure of one call (all on the caller's stream, no host sync):
//   1. mla_plan_kernel     one workgroup turns device seq_lens into a list of
//                          work items (sequence, row group, key range)
//   2. decode kernel       one workgroup per item, S^T = K Q^T and
//                          O^T += V^T P^T on bf16 MFMA with a base-2 online
//                          softmax; writes the final rows or a split partial
//                          (fp32 normalised o, base-2 lse):
//        mla_decode_narrow  <= 16 query rows per sequence (HBM-bound): every
//                           wave streams its own key tiles HBM -> LDS
//        mla_decode_wide    up to 64 / 128 rows per item (MFMA-heavy): the 4
//                           waves share 64-key tiles, each owns 16 / 32 rows
//   3. mla_combine_kernel  merges the partials of split (sequence, row group)
//                          pairs with log-sum-exp weights
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "mla_decode.h"

namespace {

constexpr int D = MLA_D_QK;          // 576
constexpr int DV = MLA_D_V;          // 512
constexpr int NT = 64;               // key granularity of split chunks
constexpr int NTHREADS = 256;        // 4 wave64 per workgroup
constexpr int OSTRIDE = DV + 4;      // fp32 row stride of the output staging
constexpr int TARGET_ITEMS = 256;    // automatic split: about one work item per CU
constexpr int MIN_CHUNK = 256;       // shortest automatic split chunk (keys)
constexpr int HEADER_BYTES = 256;
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
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// shared host/device planning arithmetic
// ---------------------------------------------------------------------------

// Row grouping: kind 0 = narrow kernel (<= 16 rows), kind 1 = wide kernel
// with 16 rows per wave (64-row items). (A wide variant with 32 rows per wave,
// 128-row items, exists as a template but does not fit the register file
// without spilling, so it is not selected.)
struct RowCfg {
  int kind;
  int rgs;     // query rows per work item
  int nrg;     // row groups per sequence
  int target;  // work items the automatic split aims for
};

__host__ __device__ inline RowCfg row_config(int rows) {
  RowCfg c;
  c.kind = rows <= 16 ? 0 : 1;
  c.rgs = c.kind == 0 ? 16 : 64;
  c.nrg = (rows + c.rgs - 1) / c.rgs;
  c.target = TARGET_ITEMS;
  return c;
}

__host__ __device__ inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Split of one sequence's key range [0, keys) into n chunks of `len` keys
// (len a multiple of the tile); keys == 0 still yields one (empty) chunk.
__host__ __device__ inline void seq_split(int keys, int chunk, int* n, int* len) {
  if (keys <= 0) { *n = 1; *len = 0; return; }
  int n0 = (keys + chunk - 1) / chunk;
  int l = round_up((keys + n0 - 1) / n0, NT);
  *len = l;
  *n = (keys + l - 1) / l;
}

__host__ __device__ inline int chunk_from_work(long long work, int forced, int target) {
  if (forced > 0) return forced;
  long long c = (work + target - 1) / target;
  c = (c + NT - 1) / NT * NT;
  if (c < MIN_CHUNK) c = MIN_CHUNK;
  if (c > (1LL << 30)) c = 1LL << 30;
  return static_cast<int>(c);
}

// Upper bound on work items (and partial slots) for a description.
inline long long max_items_bound(int batch, int rows, int max_keys, int forced) {
  RowCfg rc = row_config(rows);
  long long per_seq_cap = (max_keys + NT - 1) / NT;             // chunks are >= 64 keys
  if (forced > 0) per_seq_cap = (max_keys + forced - 1) / forced;
  if (per_seq_cap < 1) per_seq_cap = 1;
  long long cap = (long long)rc.nrg * batch * per_seq_cap;
  if (forced == 0) {
    long long auto_cap = rc.target + (long long)rc.nrg * batch;
    long long min_cap = (long long)rc.nrg * batch * ((max_keys + MIN_CHUNK - 1) / MIN_CHUNK);
    if (min_cap < (long long)rc.nrg * batch) min_cap = (long long)rc.nrg * batch;
    if (auto_cap < cap) cap = auto_cap;
    if (min_cap < cap) cap = min_cap;
  }
  return cap;
}

struct WsLayout {
  size_t items, pairs, part_lse, part_o, total;
  long long max_items;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WsLayout ws_layout(int batch, int s_q, int heads, int max_keys, int forced) {
  int rows = s_q * heads;
  RowCfg rc = row_config(rows);
  WsLayout w;
  w.max_items = max_items_bound(batch, rows, max_keys, forced);
  size_t off = HEADER_BYTES;
  w.items = off;   off = align256(off + (size_t)w.max_items * ITEM_INTS * 4);
  w.pairs = off;   off = align256(off + (size_t)batch * rc.nrg * 2 * 4);
  w.part_lse = off; off = align256(off + (size_t)w.max_items * rc.rgs * 4);
  w.part_o = off;  off = align256(off + (size_t)w.max_items * rc.rgs * DV * 4);
  w.total = off;
  return w;
}

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
  __bf16 x = static_cast<__bf16>(a);
  __bf16 y = static_cast<__bf16>(b);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, y)) << 16);
}

// Transposed 64-bit LDS read (see the V^T operand set-up in the decode kernel).
__device__ __forceinline__ s16x4_t read_vt(const char* p) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
  // generic -> LDS address space needs a C-style cast
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
}

// ---------------------------------------------------------------------------
// planner
// ---------------------------------------------------------------------------

struct PlanParams {
  const int32_t* seq_lens;
  int32_t* header;       // [0] items [1] chunk [2] slots [3] clamp flag
  int32_t* items;        // ITEM_INTS per item
  int32_t* pairs;        // per (b, row group): first slot, number of splits
  int batch, nrg, max_keys, forced_chunk, target;
  long long max_items;
};

constexpr int PLAN_THREADS = 256;
constexpr int PLAN_WAVES = PLAN_THREADS / 64;

template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    T u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  return v;
}

// One workgroup. Thread t owns the contiguous sequences [t*per, (t+1)*per);
// seq_lens are read once into LDS. Two block-wide steps: the total work
// (sum of row groups x keys rounded to 64) fixes the chunk length, then an
// exclusive scan of per-thread item / partial-slot counts places every item.
__global__ __launch_bounds__(PLAN_THREADS) void mla_plan_kernel(PlanParams p) {
  extern __shared__ int32_t s_len[];          // batch entries
  __shared__ long long s_work[PLAN_WAVES];
  __shared__ int s_items[PLAN_WAVES], s_slots[PLAN_WAVES], s_flag[PLAN_WAVES];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;

  int clamped = 0;
  for (int b = tid; b < p.batch; b += PLAN_THREADS) {
    int L = p.seq_lens[b];
    clamped |= (L < 0 || L > p.max_keys);
    s_len[b] = min(max(L, 0), p.max_keys);
  }
  __syncthreads();

  const int per = (p.batch + PLAN_THREADS - 1) / PLAN_THREADS;
  const int b0 = min(p.batch, tid * per);
  const int b1 = min(p.batch, b0 + per);
  long long work = 0;
  for (int b = b0; b < b1; ++b) work += (long long)p.nrg * round_up(s_len[b], NT);
  work = wave_inclusive_scan(work);
  const int any_clamped = __any(clamped);
  if (lane == 63) {
    s_work[wv] = work;
    s_flag[wv] = any_clamped;
  }
  __syncthreads();
  long long total = 0;
  int flag = 0;
#pragma unroll
  for (int i = 0; i < PLAN_WAVES; ++i) {
    total += s_work[i];
    flag |= s_flag[i];
  }
  const int chunk = chunk_from_work(total, p.forced_chunk, p.target);

  int my_items = 0, my_slots = 0;
  for (int b = b0; b < b1; ++b) {
    int n, len;
    seq_split(s_len[b], chunk, &n, &len);
    my_items += p.nrg * n;
    if (n > 1) my_slots += p.nrg * n;
  }
  const int inc_items = wave_inclusive_scan(my_items);
  const int inc_slots = wave_inclusive_scan(my_slots);
  if (lane == 63) {
    s_items[wv] = inc_items;
    s_slots[wv] = inc_slots;
  }
  __syncthreads();
  int item = inc_items - my_items, slot = inc_slots - my_slots;
  int tot_items = 0, tot_slots = 0;
#pragma unroll
  for (int i = 0; i < PLAN_WAVES; ++i) {
    if (i < wv) {
      item += s_items[i];
      slot += s_slots[i];
    }
    tot_items += s_items[i];
    tot_slots += s_slots[i];
  }

  for (int b = b0; b < b1; ++b) {
    const int L = s_len[b];
    int n, len;
    seq_split(L, chunk, &n, &len);
    for (int rg = 0; rg < p.nrg; ++rg) {
      p.pairs[2 * (b * p.nrg + rg)] = n > 1 ? slot : -1;
      p.pairs[2 * (b * p.nrg + rg) + 1] = n;
      for (int s = 0; s < n; ++s) {
        if (item < p.max_items) {
          int4* it = reinterpret_cast<int4*>(p.items + (size_t)item * ITEM_INTS);
          it[0] = make_int4(b, rg, s * len, min(L, (s + 1) * len));
          it[1] = make_int4(n > 1 ? slot + s : -1, 0, 0, 0);
        }
        ++item;
      }
      if (n > 1) slot += n;
    }
  }
  if (tid == 0) {
    p.header[0] = (int)min((long long)tot_items, p.max_items);
    p.header[1] = chunk;
    p.header[2] = tot_slots;
    p.header[3] = flag;
  }
}

// ---------------------------------------------------------------------------
// decode kernel
// ---------------------------------------------------------------------------

struct FwdParams {
  const uint16_t* q;
  const uint8_t* kv;
  const int32_t* block_table;
  const int32_t* seq_lens;
  uint16_t* out;
  float* lse;
  const int32_t* header;
  const int32_t* items;
  float* part_o;
  float* part_lse;
  int heads, s_q, rows, bs, max_blocks, max_keys, causal, num_blocks;
  float scale_log2;   // softmax_scale * kv_scale * log2(e)
  float out_scale;    // kv_scale
};

// Final step of a work item. Each of the 4 waves holds, for the 16 rows of its
// row tile (one row per lane, lane groups splitting the dims), the running max
// m (base 2), its share of the running sum, and unnormalised O^T. The KS
// waves that share a row tile are merged through LDS (weights 2^(m_k - M)),
// then the rows are written as final bf16 out + natural-log lse (slot < 0), or
// as an fp32 split partial (normalised o and base-2 lse). Every wave must be
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

  constexpr int TPR = NTHREADS / RGS;   // threads per row
  constexpr int DPT = DV / TPR;         // dims per thread
  const int rr = tid / TPR;             // row within the item
  const int d0 = (tid % TPR) * DPT;
  const int rtile = rr / 16, rc = rr % 16;
  float mk[KS], wk[KS];
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    mk[k] = mls[((rtile * KS + k) * 16 + rc) * 2];
    M = fmaxf(M, mk[k]);
  }
  float lsum = 0.f;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    wk[k] = mk[k] == -INFINITY ? 0.f : exp2f(mk[k] - M);
    lsum += wk[k] * mls[((rtile * KS + k) * 16 + rc) * 2 + 1];
  }
  const int grow = rg * RGS + rr;
  const bool row_ok = grow < p.rows;
  const bool empty = !(lsum > 0.f);
  const float inv = empty ? 0.f : p.out_scale / lsum;
  const float lse2 = empty ? -INFINITY : M + log2f(lsum);
  const size_t orow = (size_t)b * p.rows + grow;

  if (slot < 0 && row_ok) {
    uint16_t* dst = p.out + orow * DV + d0;
#pragma unroll
    for (int d = 0; d < DPT; d += 8) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < KS; ++k)
          s += wk[k] * ost[((rtile * KS + k) * 16 + rc) * OSTRIDE + d0 + d + e];
        acc[e] = s * inv;
      }
      *reinterpret_cast<uint4*>(dst + d) =
          make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    }
    if (p.lse != nullptr && (tid % TPR) == 0) p.lse[orow] = lse2 * LN2;
  } else if (slot >= 0 && row_ok) {
    float* dst = p.part_o + ((size_t)slot * RGS + rr) * DV + d0;
#pragma unroll
    for (int d = 0; d < DPT; d += 4) {
      f32x4_t acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < KS; ++k)
          s += wk[k] * ost[((rtile * KS + k) * 16 + rc) * OSTRIDE + d0 + d + e];
        acc[e] = s * inv;
      }
      *reinterpret_cast<f32x4_t*>(dst + d) = acc;
    }
    if ((tid % TPR) == 0) p.part_lse[(size_t)slot * RGS + rr] = lse2;
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
// side is always 64 consecutive 16-byte slots.

constexpr int H16_KT = 16;                      // keys per wave tile
constexpr int H16_TILE = H16_KT * D * 2;        // 18432 bytes (bf16)
constexpr int H16_DMA = H16_TILE / 1024;        // 18 wave-wide 1 KB transfers
constexpr int H16_GSTRIDE = H16_KT * 128;       // bytes per 128-byte column group

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

// fp8 tiles: 32 keys x 576 bytes = 18432 bytes, laid out as
// [9 column groups of 64 B][32 keys][4 x 16-byte chunks] with the chunk
// position XOR-swizzled by f(key) = ((key >> 2) + (key >> 4)) & 3, which keeps
// both the 8-byte K reads and the 8-bit transposed V reads spread over banks.
constexpr int F8_KT = 32;
constexpr int F8_GSTRIDE = F8_KT * 64;

__device__ __forceinline__ int f8_swz(int key) { return ((key >> 2) + (key >> 4)) & 3; }

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

  const int n_items = p.header[0];
  const int item_id = blockIdx.x;
  if (item_id >= n_items) return;
  const int32_t* it = p.items + (size_t)item_id * ITEM_INTS;
  // work-item fields are uniform: keep them (and all tile addressing derived
  // from them) in SGPRs, so no vector load ever enters the DMA vmcnt queue
  const int b = __builtin_amdgcn_readfirstlane(it[0]);
  const int t0 = __builtin_amdgcn_readfirstlane(it[2]);
  const int t1 = __builtin_amdgcn_readfirstlane(it[3]);
  const int slot = __builtin_amdgcn_readfirstlane(it[4]);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c16 = lane & 15;

  const int L = __builtin_amdgcn_readfirstlane(min(max(p.seq_lens[b], 0), p.max_keys));
  const int row = c16;
  const bool row_ok = row < p.rows;
  int limit = 0;
  if (row_ok) {
    int tok = row / p.heads;
    int vis = p.causal ? L - p.s_q + 1 + tok : L;
    limit = min(vis, t1);
  }

  bf16x8_t qb[D / 32];
  {
    const uint16_t* qrow = p.q + ((size_t)b * p.rows + (row_ok ? row : 0)) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * g)
                       : make_uint4(0, 0, 0, 0);
      qb[s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  // Consume the q loads here, so the compiler's own vmcnt wait for them sits
  // before the first DMA and not inside the tile loop (it cannot see the DMAs).
#pragma unroll
  for (int s = 0; s < D / 32; ++s) asm volatile("" ::"v"(qb[s]));

  f32x4_t o[DV / 16];
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  // ---- lane constants (LDS byte offsets inside a tile, DMA source offsets) ----
  uint32_t dma_lane[2];
  int kb[2][2];   // K operand: [M tile][s & 1], add (s >> 1) * column-group stride
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
    // position lane & 3; f(key) = ((lane >> 4) + (n & 1)) & 3.
#pragma unroll
    for (int h = 0; h < 2; ++h)
      dma_lane[h] = (lane >> 2) * ROWB + (((lane & 3) ^ (((lane >> 4) + h) & 3)) << 4);
    // K: key 16*mi + c16, bytes 32*s + 8*g -> chunk 2*s + (g >> 1), half g & 1
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        kb[mi][h] = (16 * mi + c16) * 64 +
                    (((2 * h + (g >> 1)) ^ f8_swz(16 * mi + c16)) << 4) + (g & 1) * 8;
    // V^T: lane s = 2*jj + q supplies V[key_jj][16*dt + 8*q ..+7] with key_jj =
    // 4g + jj (jj < 4) or 16 + 4g + jj - 4, so ds_read_b64_tr_b8 hands lane
    // c16 the 8 values V[key_0..7][16*dt + c16].
    const int jj = c16 >> 1, q = c16 & 1;
    const int key = jj < 4 ? 4 * g + jj : 16 + 4 * g + (jj - 4);
#pragma unroll
    for (int c = 0; c < 4; ++c) vt[c] = key * 64 + ((c ^ f8_swz(key)) << 4) + q * 8;
  }
  constexpr int GSTRIDE = F8 ? F8_GSTRIDE : H16_GSTRIDE;

  // The block table is read-only for the whole kernel: reading it through the
  // constant address space keeps these uniform loads on the scalar unit, so
  // they never enter the vmcnt queue the DMA waits below count on.
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const_i32* bt = (const_i32*)(p.block_table + (size_t)b * p.max_blocks);
  char* wbuf = smem + w * 2 * H16_TILE;
  const int ntiles = (t1 - t0 + KT - 1) / KT;

  // Issue the NDMA transfers of tile j into dst (always NDMA VMEM
  // instructions, so the vmcnt arithmetic below is exact). Keys past the end
  // are fetched from a valid row of the page and zeroed after arrival.
  auto issue = [&](int j, char* dst) {
    const int ts = t0 + KT * j;
    int page = bt[ts / p.bs];
    if (page < 0 || page >= p.num_blocks) page = 0;
    const char* src = reinterpret_cast<const char*>(p.kv) + ((size_t)page * p.bs + (ts % p.bs)) * ROWB;
    const uint32_t l0 = lds_addr(dst);
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
      if constexpr (!F8)
        lds_dma16_nt(src + (n & 1) * 8 * ROWB + (n >> 1) * 128, dma_lane[0], l0 + n * 1024);
      else
        lds_dma16(src + (n & 1) * 16 * ROWB + (n >> 1) * 64, dma_lane[n & 1], l0 + n * 1024);
    }
  };
  auto valid_keys = [&](int j) {
    const int ts = t0 + KT * j;
    int page = bt[ts / p.bs];
    if (page < 0 || page >= p.num_blocks) return 0;
    return min(KT, t1 - ts);
  };
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
    fix_tail(valid_keys(j), cur);
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
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        bf16x8_t a;
        if constexpr (!F8)
          a = *reinterpret_cast<const bf16x8_t*>(cur + kb[mi][s & 1] + (s >> 1) * GSTRIDE);
        else
          a = fp8x8_to_bf16x8_v(*reinterpret_cast<const uint2*>(cur + kb[mi][s & 1] + (s >> 1) * GSTRIDE));
        sacc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[s], sacc[mi], 0, 0, 0);
      }
    }

    float x[MT][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int key = ts + 16 * mi + 4 * g + jj;
        float v = sacc[mi][jj] * p.scale_log2;
        v = key < limit ? v : -INFINITY;
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
  if (w < ntiles) issue(w, wbuf);
  for (; j < ntiles; j += 4, ++itn) {
    cur = prepare(j, itn);
    if (!compute(cur, t0 + KT * j, std::false_type{})) break;
  }
  if (j < ntiles) {   // rare: finish with rescaling, starting at the resident tile j
    compute(cur, t0 + KT * j, std::true_type{});
    for (j += 4, ++itn; j < ntiles; j += 4, ++itn)
      compute(prepare(j, itn), t0 + KT * j, std::true_type{});
  }
  __syncthreads();
  merge_and_store<4>(p, smem, o, m_run, l_run, b, 0, slot);
}

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

  const int n_items = p.header[0];
  const int item_id = blockIdx.x;
  if (item_id >= n_items) return;
  const int32_t* it = p.items + (size_t)item_id * ITEM_INTS;
  // uniform work-item fields, pinned to SGPRs (see the narrow kernel)
  const int b = __builtin_amdgcn_readfirstlane(it[0]);
  const int rg = __builtin_amdgcn_readfirstlane(it[1]);
  const int t0 = __builtin_amdgcn_readfirstlane(it[2]);
  const int t1 = __builtin_amdgcn_readfirstlane(it[3]);
  const int slot = __builtin_amdgcn_readfirstlane(it[4]);

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
      uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * g)
                       : make_uint4(0, 0, 0, 0);
      qb[s] = __builtin_bit_cast(bf16x8_t, v);
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
  const int ntiles = (t1 - t0 + W_NTK - 1) / W_NTK;
  // fp8 tiles are fetched by waves 0 and 1 only (18 transfers per tile)
  const bool dma_wave = !F8 || w < 2;

  // Issue this wave's NDMA transfers of tile j (exactly NDMA VMEM
  // instructions per participating wave; vmcnt arithmetic relies on it).
  auto issue = [&](int j) {
    const int ts = t0 + W_NTK * j;
    int page = bt[ts / p.bs];
    if (page < 0 || page >= p.num_blocks) page = 0;
    const char* src = reinterpret_cast<const char*>(p.kv) + ((size_t)page * p.bs + (ts % p.bs)) * ROWB;
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
  auto valid_keys = [&](int j) {
    const int ts = t0 + W_NTK * j;
    int page = bt[ts / p.bs];
    if (page < 0 || page >= p.num_blocks) return 0;
    return min(W_NTK, t1 - ts);
  };
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
    f32x4_t sacc[2][2];   // [M tile][even/odd k-step]: four independent chains
#pragma unroll
    for (int h = 0; h < 2; ++h) sacc[h][0] = sacc[h][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(cur + kb[h][s & 1] + (s >> 1) * W_GSTRIDE);
        sacc[h][s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[s], sacc[h][s & 1], 0, 0, 0);
      }
    }

    // ---- online softmax (lane = one row, 8 keys) ----
    float x[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int key = ts + 16 * h + 4 * g + jj;
        float v = (sacc[h][0][jj] + sacc[h][1][jj]) * p.scale_log2;
        v = key < limit ? v : -INFINITY;
        x[h][jj] = v;
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
    float e[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        e[h][jj] = m_run == -INFINITY ? 0.f : exp2f(x[h][jj] - m_run);
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

  // ---- write this wave's rows: final (slot < 0) or split partial ----
  const float l_row = wave_sum_across_groups(l_run);
  if (row_ok) {
    const bool empty = !(l_row > 0.f);
    const float inv = empty ? 0.f : p.out_scale / l_row;
    const float lse2 = empty ? -INFINITY : m_run + log2f(l_row);
    const size_t orow = (size_t)b * p.rows + row;
    if (slot < 0) {
      uint16_t* dst = p.out + orow * DV + 4 * g;
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) {
        const f32x4_t v = o[dt] * inv;
        *reinterpret_cast<uint2*>(dst + 16 * dt) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
      if (p.lse != nullptr && g == 0) p.lse[orow] = lse2 * LN2;
    } else {
      float* dst = p.part_o + ((size_t)slot * RGS + row_local) * DV + 4 * g;
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt)
        *reinterpret_cast<f32x4_t*>(dst + 16 * dt) = o[dt] * inv;
      if (g == 0) p.part_lse[(size_t)slot * RGS + row_local] = lse2;
    }
  }
}

// ---------------------------------------------------------------------------
// combine kernel
// ---------------------------------------------------------------------------

struct CombineParams {
  const int32_t* pairs;
  const float* part_o;
  const float* part_lse;
  uint16_t* out;
  float* lse;
  int rows, rgs, nrg, n_pairs;
};

// Grid (pair, chunk): thread (row, 8-dim slice) of one (sequence, row group)
// pair; only pairs that were split do work. Merge of the pair's n partials:
// lse = log2(sum_s 2^lse_s), out = sum_s 2^(lse_s - lse) o_s.
constexpr int COMBINE_SLICES = DV / 8;   // 64 threads per row

__global__ __launch_bounds__(NTHREADS) void mla_combine_kernel(CombineParams p) {
  const int pair = blockIdx.x;
  const int first = p.pairs[2 * pair];
  const int n = p.pairs[2 * pair + 1];
  if (first < 0 || n <= 1) return;
  const int idx = blockIdx.y * NTHREADS + threadIdx.x;
  const int rr = idx / COMBINE_SLICES;
  const int d0 = (idx % COMBINE_SLICES) * 8;
  const int b = pair / p.nrg, rg = pair % p.nrg;
  const int grow = rg * p.rgs + rr;
  if (rr >= p.rgs || grow >= p.rows) return;

  const float* lse_s = p.part_lse + (size_t)first * p.rgs + rr;
  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, lse_s[(size_t)s * p.rgs]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  const float* src = p.part_o + ((size_t)first * p.rgs + rr) * DV + d0;
  const size_t sstride = (size_t)p.rgs * DV;
  int s = 0;
  for (; s + 2 <= n; s += 2) {   // two splits per step: four 16-byte loads in flight
    const float l0 = lse_s[(size_t)s * p.rgs], l1 = lse_s[(size_t)(s + 1) * p.rgs];
    const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(src + s * sstride);
    const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(src + s * sstride + 4);
    const f32x4_t c0 = *reinterpret_cast<const f32x4_t*>(src + (s + 1) * sstride);
    const f32x4_t c1 = *reinterpret_cast<const f32x4_t*>(src + (s + 1) * sstride + 4);
    const float w0 = l0 == -INFINITY ? 0.f : exp2f(l0 - M);
    const float w1 = l1 == -INFINITY ? 0.f : exp2f(l1 - M);
    den += w0 + w1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += w0 * a0[e] + w1 * c0[e];
      acc[4 + e] += w0 * a1[e] + w1 * c1[e];
    }
  }
  if (s < n) {
    const float l0 = lse_s[(size_t)s * p.rgs];
    const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(src + s * sstride);
    const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(src + s * sstride + 4);
    const float w0 = l0 == -INFINITY ? 0.f : exp2f(l0 - M);
    den += w0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += w0 * a0[e];
      acc[4 + e] += w0 * a1[e];
    }
  }
  const bool empty = !(den > 0.f);
  const float inv = empty ? 0.f : 1.f / den;
  const size_t orow = (size_t)b * p.rows + grow;
  *reinterpret_cast<uint4*>(p.out + orow * DV + d0) =
      make_uint4(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                 pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv));
  if (p.lse != nullptr && d0 == 0) p.lse[orow] = empty ? -INFINITY : (M + log2f(den)) * LN2;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

mla_status_t check_desc(int32_t s_q, const mla_decode_desc_t* d) {
  if (d == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (d->batch < 0 || d->num_heads < 1 || s_q < 1 || d->num_blocks < 1 ||
      d->max_blocks_per_seq < 1 || d->split_keys < 0 || (d->causal != 0 && d->causal != 1))
    return MLA_ERR_INVALID_ARGUMENT;
  if (d->num_heads > MLA_MAX_HEADS || s_q > MLA_MAX_SQ || d->batch > MLA_MAX_BATCH)
    return MLA_ERR_UNSUPPORTED;
  if (d->block_size != 64 && d->block_size != 128) return MLA_ERR_UNSUPPORTED;
  if (d->kv_dtype != MLA_DTYPE_BF16 && d->kv_dtype != MLA_DTYPE_FP8_E4M3FN) return MLA_ERR_UNSUPPORTED;
  if (d->split_keys % NT != 0) return MLA_ERR_INVALID_ARGUMENT;
  long long max_keys = (long long)d->max_blocks_per_seq * d->block_size;
  if (max_keys > (1LL << 30)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

int max_keys_of(const mla_decode_desc_t* d) { return d->max_blocks_per_seq * d->block_size; }

template <int KVT>
void launch_decode(int kind, dim3 grid, hipStream_t st, const FwdParams& fp) {
  switch (kind) {
    case 0: hipLaunchKernelGGL((mla_decode_narrow<KVT>), grid, dim3(NTHREADS), 0, st, fp); break;
    default: hipLaunchKernelGGL((mla_decode_wide<KVT, 1>), grid, dim3(NTHREADS), 0, st, fp); break;
  }
}

mla_status_t launch_plan(const int32_t* seq_lens, int32_t s_q, const mla_decode_desc_t* desc,
                         void* workspace, const WsLayout& ws, hipStream_t st) {
  RowCfg rc = row_config(s_q * desc->num_heads);
  char* base = static_cast<char*>(workspace);
  PlanParams pp;
  pp.seq_lens = seq_lens;
  pp.header = reinterpret_cast<int32_t*>(base);
  pp.items = reinterpret_cast<int32_t*>(base + ws.items);
  pp.pairs = reinterpret_cast<int32_t*>(base + ws.pairs);
  pp.batch = desc->batch;
  pp.nrg = rc.nrg;
  pp.target = rc.target;
  pp.max_keys = max_keys_of(desc);
  pp.forced_chunk = desc->split_keys;
  pp.max_items = ws.max_items;
  hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(PLAN_THREADS),
                     static_cast<unsigned>(desc->batch) * sizeof(int32_t), st, pp);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

}  // namespace

extern "C" {

size_t mla_decode_workspace_size(int32_t s_q, const mla_decode_desc_t* desc) {
  if (check_desc(s_q, desc) != MLA_OK) return 0;
  return ws_layout(desc->batch, s_q, desc->num_heads, max_keys_of(desc), desc->split_keys).total;
}

mla_status_t mla_decode_plan(const int32_t* seq_lens, int32_t s_q, const mla_decode_desc_t* desc,
                             void* workspace, size_t workspace_bytes, void* stream) {
  mla_status_t st = check_desc(s_q, desc);
  if (st != MLA_OK) return st;
  if (seq_lens == nullptr || workspace == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (!aligned(seq_lens, 4) || !aligned(workspace, 256)) return MLA_ERR_INVALID_ARGUMENT;
  WsLayout ws = ws_layout(desc->batch, s_q, desc->num_heads, max_keys_of(desc), desc->split_keys);
  if (workspace_bytes < ws.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (desc->batch == 0) return MLA_OK;
  return launch_plan(seq_lens, s_q, desc, workspace, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

mla_status_t check_call(const void* q, const void* kv_cache, const int32_t* block_table,
                        const int32_t* seq_lens, int32_t s_q, float softmax_scale,
                        float kv_scale, const void* out, const float* lse,
                        const mla_decode_desc_t* desc, const void* workspace,
                        size_t workspace_bytes, WsLayout* ws) {
  mla_status_t st = check_desc(s_q, desc);
  if (st != MLA_OK) return st;
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f) ||
      !(std::isfinite(kv_scale) && kv_scale > 0.f))
    return MLA_ERR_INVALID_ARGUMENT;
  if (q == nullptr || kv_cache == nullptr || block_table == nullptr || seq_lens == nullptr ||
      out == nullptr || workspace == nullptr)
    return MLA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(workspace, 256) ||
      (lse != nullptr && !aligned(lse, 4)))
    return MLA_ERR_INVALID_ARGUMENT;
  *ws = ws_layout(desc->batch, s_q, desc->num_heads, max_keys_of(desc), desc->split_keys);
  if (workspace_bytes < ws->total) return MLA_ERR_WORKSPACE_TOO_SMALL;
  return MLA_OK;
}

mla_status_t launch_decode_kernel(const void* q, const void* kv_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    int32_t s_q, float softmax_scale, float kv_scale, void* out,
                                    float* lse, const mla_decode_desc_t* desc, void* workspace,
                                    const WsLayout& ws, hipStream_t hs, bool combine) {
  const int rows = s_q * desc->num_heads;
  RowCfg rc = row_config(rows);
  char* base = static_cast<char*>(workspace);
  FwdParams fp;
  fp.q = static_cast<const uint16_t*>(q);
  fp.kv = static_cast<const uint8_t*>(kv_cache);
  fp.block_table = block_table;
  fp.seq_lens = seq_lens;
  fp.out = static_cast<uint16_t*>(out);
  fp.lse = lse;
  fp.header = reinterpret_cast<const int32_t*>(base);
  fp.items = reinterpret_cast<const int32_t*>(base + ws.items);
  fp.part_o = reinterpret_cast<float*>(base + ws.part_o);
  fp.part_lse = reinterpret_cast<float*>(base + ws.part_lse);
  fp.heads = desc->num_heads;
  fp.s_q = s_q;
  fp.rows = rows;
  fp.bs = desc->block_size;
  fp.max_blocks = desc->max_blocks_per_seq;
  fp.max_keys = max_keys_of(desc);
  fp.causal = desc->causal;
  fp.num_blocks = desc->num_blocks;
  fp.scale_log2 = softmax_scale * kv_scale * LOG2E;
  fp.out_scale = kv_scale;
  dim3 grid(static_cast<unsigned>(ws.max_items));
  if (desc->kv_dtype == MLA_DTYPE_BF16)
    launch_decode<MLA_DTYPE_BF16>(rc.kind, grid, hs, fp);
  else
    launch_decode<MLA_DTYPE_FP8_E4M3FN>(rc.kind, grid, hs, fp);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  if (!combine) return MLA_OK;

  CombineParams cp;
  cp.pairs = reinterpret_cast<const int32_t*>(base + ws.pairs);
  cp.part_o = fp.part_o;
  cp.part_lse = fp.part_lse;
  cp.out = fp.out;
  cp.lse = lse;
  cp.rows = rows;
  cp.rgs = rc.rgs;
  cp.nrg = rc.nrg;
  cp.n_pairs = desc->batch * rc.nrg;
  const unsigned chunks = (unsigned)((rc.rgs * COMBINE_SLICES + NTHREADS - 1) / NTHREADS);
  hipLaunchKernelGGL(mla_combine_kernel, dim3(cp.n_pairs, chunks), dim3(NTHREADS), 0, hs, cp);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status_t mla_decode(const void* q, const void* kv_cache, const int32_t* block_table,
                        const int32_t* seq_lens, int32_t s_q, float softmax_scale,
                        float kv_scale, void* out, float* lse, const mla_decode_desc_t* desc,
                        void* workspace, size_t workspace_bytes, void* stream) {
  WsLayout ws;
  mla_status_t st = check_call(q, kv_cache, block_table, seq_lens, s_q, softmax_scale, kv_scale,
                               out, lse, desc, workspace, workspace_bytes, &ws);
  if (st != MLA_OK) return st;
  if (desc->batch == 0) return MLA_OK;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  st = launch_plan(seq_lens, s_q, desc, workspace, ws, hs);
  if (st != MLA_OK) return st;
  return launch_decode_kernel(q, kv_cache, block_table, seq_lens, s_q, softmax_scale, kv_scale,
                                out, lse, desc, workspace, ws, hs, true);
}

mla_status_t mla_decode_fwd_only(const void* q, const void* kv_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, int32_t s_q, float softmax_scale,
                                 float kv_scale, void* out, float* lse,
                                 const mla_decode_desc_t* desc, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  WsLayout ws;
  mla_status_t st = check_call(q, kv_cache, block_table, seq_lens, s_q, softmax_scale, kv_scale,
                               out, lse, desc, workspace, workspace_bytes, &ws);
  if (st != MLA_OK) return st;
  if (desc->batch == 0) return MLA_OK;
  return launch_decode_kernel(q, kv_cache, block_table, seq_lens, s_q, softmax_scale, kv_scale,
                                out, lse, desc, workspace, ws, static_cast<hipStream_t>(stream),
                                false);
}

int32_t mla_plan_host(const int32_t* seq_lens_host, int32_t s_q, const mla_decode_desc_t* desc,
                      int32_t* items, int32_t max_items, int32_t* rows_per_item,
                      int32_t* chunk_keys) {
  if (check_desc(s_q, desc) != MLA_OK || (desc->batch > 0 && seq_lens_host == nullptr))
    return -1;
  RowCfg rc = row_config(s_q * desc->num_heads);
  const int max_keys = max_keys_of(desc);
  long long work = 0;
  for (int b = 0; b < desc->batch; ++b) {
    int L = std::min(std::max(seq_lens_host[b], 0), max_keys);
    work += (long long)rc.nrg * round_up(L, NT);
  }
  const int chunk = chunk_from_work(work, desc->split_keys, rc.target);
  if (rows_per_item) *rows_per_item = rc.rgs;
  if (chunk_keys) *chunk_keys = chunk;
  int item = 0, slot = 0;
  for (int b = 0; b < desc->batch; ++b) {
    int L = std::min(std::max(seq_lens_host[b], 0), max_keys);
    int n, len;
    seq_split(L, chunk, &n, &len);
    for (int rg = 0; rg < rc.nrg; ++rg) {
      for (int s = 0; s < n; ++s) {
        if (item >= max_items) return -1;
        if (items) {
          int32_t* it = items + (size_t)item * ITEM_INTS;
          it[0] = b; it[1] = rg; it[2] = s * len; it[3] = std::min(L, (s + 1) * len);
          it[4] = n > 1 ? slot + s : -1; it[5] = 0; it[6] = 0; it[7] = 0;
        }
        ++item;
      }
      if (n > 1) slot += n;
    }
  }
  return item;
}

const char* mla_status_string(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARGUMENT: return "MLA_ERR_INVALID_ARGUMENT";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

}  // extern "C"
