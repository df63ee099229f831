// Paged MLA decode for MI355X (gfx950 / CDNA4): split planner, MFMA decode
// kernel and LSE combine, behind the C ABI declared in include/mla_decode.h.
//
// Operation: decode attention of MLA in its MQA form ("[WIP][Attention]
// FlashAttn MLA", description) with d = 576, dv = 512, one KV head, a paged
// cache in bf16 or fp8 e4m3fn ("[Attention] Blackwell FP8 MLA support with
// CUTLASS_MLA backend", review thread: the kernel test's parameters).
//
// Structure of one call (all on the caller's stream, no host sync):
//   1. mla_plan_kernel     one workgroup turns device seq_lens into a list of
//                          work items (sequence, row group, key range)
//   2. mla_decode_fwd      one workgroup per item: page-table gather of 64-key
//                          tiles into LDS (fp8 dequantised to bf16 on the way),
//                          S^T = K Q^T and O^T += V^T P^T on MFMA, online
//                          softmax in base 2, write of the final row or of a
//                          split partial (fp32 o, base-2 lse)
//   3. mla_combine_kernel  merges the partials of split (sequence, row group)
//                          pairs with log-sum-exp weights
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "mla_decode.h"

namespace {

constexpr int D = MLA_D_QK;          // 576
constexpr int DV = MLA_D_V;          // 512
constexpr int NT = 64;               // keys per LDS tile
constexpr int NTHREADS = 256;        // 4 wave64 per workgroup
constexpr int CHUNKS = D / 8;        // 72 16-byte bf16 chunks per row
constexpr int TILE_BYTES = NT * D * 2;            // 73728: one bf16 tile
constexpr int OSTRIDE = DV + 4;      // fp32 row stride of the output staging
constexpr int TARGET_ITEMS_WIDE = 512;   // row groups of 32/64 rows: ~2 items per CU
constexpr int TARGET_ITEMS_NARROW = 256; // <= 16 rows: one 4-wave item per CU
constexpr int MIN_CHUNK = 256;       // shortest automatic split chunk (keys)
constexpr int HEADER_BYTES = 256;
constexpr int ITEM_INTS = 8;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_SLACK = 8.0f;   // base-2 headroom before the running max moves

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// shared host/device planning arithmetic
// ---------------------------------------------------------------------------

struct RowCfg {
  int ks;      // waves that split each tile's keys (4, 2 or 1)
  int rgs;     // query rows per work item = 16 * (4 / ks)
  int nrg;     // row groups per sequence
  int target;  // work items the automatic split aims for
};

__host__ __device__ inline RowCfg row_config(int rows) {
  RowCfg c;
  c.ks = rows <= 16 ? 4 : (rows <= 32 ? 2 : 1);
  c.rgs = 16 * (4 / c.ks);
  c.nrg = (rows + c.rgs - 1) / c.rgs;
  c.target = rows <= 16 ? TARGET_ITEMS_NARROW : TARGET_ITEMS_WIDE;
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

// Byte offset of 16-byte chunk c (0..71) of tile row `key` in the LDS tile.
// Rows are grouped by 128-byte column group; inside a group the eight chunks
// of a row are XOR-swizzled by the row's low three bits, so the 8 lanes that
// read one chunk column of 8 consecutive rows hit 8 different bank groups.
__device__ __forceinline__ int lds_off(int key, int c) {
  return (((c >> 3) * NT + key) << 7) + ((((c & 7) ^ (key & 7))) << 4);
}

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

__global__ __launch_bounds__(PLAN_THREADS) void mla_plan_kernel(PlanParams p) {
  __shared__ long long red[PLAN_THREADS];
  __shared__ int scan_items[PLAN_THREADS];
  __shared__ int scan_slots[PLAN_THREADS];
  __shared__ int s_chunk;
  __shared__ int s_flag;
  const int tid = threadIdx.x;
  const int per = (p.batch + PLAN_THREADS - 1) / PLAN_THREADS;
  const int b0 = tid * per;
  const int b1 = min(p.batch, b0 + per);

  long long work = 0;
  int clamped = 0;
  for (int b = b0; b < b1; ++b) {
    int L = p.seq_lens[b];
    if (L < 0 || L > p.max_keys) clamped = 1;
    L = min(max(L, 0), p.max_keys);
    work += (long long)p.nrg * round_up(L, NT);
  }
  red[tid] = work;
  if (tid == 0) s_flag = 0;
  __syncthreads();
  if (clamped) atomicOr(&s_flag, 1);
  __syncthreads();
  for (int s = PLAN_THREADS / 2; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  if (tid == 0) s_chunk = chunk_from_work(red[0], p.forced_chunk, p.target);
  __syncthreads();
  const int chunk = s_chunk;

  int my_items = 0, my_slots = 0;
  for (int b = b0; b < b1; ++b) {
    int L = min(max(p.seq_lens[b], 0), p.max_keys);
    int n, len;
    seq_split(L, chunk, &n, &len);
    my_items += p.nrg * n;
    if (n > 1) my_slots += p.nrg * n;
  }
  scan_items[tid] = my_items;
  scan_slots[tid] = my_slots;
  __syncthreads();
  // inclusive Hillis-Steele scan over the 256 per-thread counts
  for (int off = 1; off < PLAN_THREADS; off <<= 1) {
    int a = tid >= off ? scan_items[tid - off] : 0;
    int c = tid >= off ? scan_slots[tid - off] : 0;
    __syncthreads();
    scan_items[tid] += a;
    scan_slots[tid] += c;
    __syncthreads();
  }
  int item = scan_items[tid] - my_items;
  int slot = scan_slots[tid] - my_slots;
  for (int b = b0; b < b1; ++b) {
    int L = min(max(p.seq_lens[b], 0), p.max_keys);
    int n, len;
    seq_split(L, chunk, &n, &len);
    for (int rg = 0; rg < p.nrg; ++rg) {
      int first = n > 1 ? slot : -1;
      p.pairs[2 * (b * p.nrg + rg)] = first;
      p.pairs[2 * (b * p.nrg + rg) + 1] = n;
      for (int s = 0; s < n; ++s) {
        if (item < p.max_items) {
          int32_t* it = p.items + (size_t)item * ITEM_INTS;
          it[0] = b;
          it[1] = rg;
          it[2] = s * len;
          it[3] = min(L, (s + 1) * len);
          it[4] = n > 1 ? slot + s : -1;
          it[5] = 0; it[6] = 0; it[7] = 0;
        }
        ++item;
      }
      if (n > 1) slot += n;
    }
  }
  if (tid == PLAN_THREADS - 1) {
    p.header[0] = (int)min((long long)scan_items[PLAN_THREADS - 1], p.max_items);
    p.header[1] = chunk;
    p.header[2] = scan_slots[PLAN_THREADS - 1];
    p.header[3] = s_flag;
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

template <int KVT>
struct TileStage;

// bf16 cache: 18 x 16 bytes per thread per 64-key tile (73728 bytes).
template <>
struct TileStage<MLA_DTYPE_BF16> {
  static constexpr int N = TILE_BYTES / 16 / NTHREADS;   // 18
  uint4 v[N];
  __device__ __forceinline__ void load(const uint8_t* src, int n_valid, int tid) {
    const uint4* s = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      int qi = j * NTHREADS + tid;
      int key = qi / CHUNKS;
      v[j] = key < n_valid ? s[qi] : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      int qi = j * NTHREADS + tid;
      int key = qi / CHUNKS;
      int c = qi - key * CHUNKS;
      *reinterpret_cast<uint4*>(lds + lds_off(key, c)) = v[j];
    }
  }
};

// fp8 cache: 9 x 16 bytes (16 codes) per thread per tile (36864 bytes),
// widened to bf16 when written to LDS.
template <>
struct TileStage<MLA_DTYPE_FP8_E4M3FN> {
  static constexpr int N = NT * D / 16 / NTHREADS;   // 9
  uint4 v[N];
  __device__ __forceinline__ void load(const uint8_t* src, int n_valid, int tid) {
    const uint4* s = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      int qi = j * NTHREADS + tid;
      int key = qi / (CHUNKS / 2);
      v[j] = key < n_valid ? s[qi] : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      int qi = j * NTHREADS + tid;
      int key = qi / (CHUNKS / 2);
      int c = 2 * (qi - key * (CHUNKS / 2));
      *reinterpret_cast<uint4*>(lds + lds_off(key, c)) = fp8x8_to_bf16x8(v[j].x, v[j].y);
      *reinterpret_cast<uint4*>(lds + lds_off(key, c + 1)) = fp8x8_to_bf16x8(v[j].z, v[j].w);
    }
  }
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
  if (grow >= p.rows) return;
  const bool empty = !(lsum > 0.f);
  const float inv = empty ? 0.f : p.out_scale / lsum;
  const float lse2 = empty ? -INFINITY : M + log2f(lsum);
  const size_t orow = (size_t)b * p.rows + grow;

  if (slot < 0) {
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
  } else {
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

// One workgroup = 4 waves handles one work item: `rgs` query rows of one
// sequence over keys [t0, t1). Wave w owns rows 16*(w / KS) .. +15 of the
// item and keys [(w % KS) * 64/KS, +64/KS) of every 64-key tile. Each wave
// keeps its own running max / sum / O^T; the KS partial states of a row tile
// are merged through LDS at the end.
//
// MFMA formulation (16x16 output tiles, lane l: column l%16, rows 4*(l/16)+j):
//   S^T[key, row] = K[key, :] . Q^T[:, row]   A = K from LDS, B = Q^T in VGPRs
//   O^T[dim, row] += V^T[dim, key] P^T[key, row]
// so each lane owns one query row (l%16) and the softmax statistics never
// leave the lane except for a max over the 4 lane groups; the S^T accumulator
// already has the layout of the P^T operand of the next product.
template <int KVT, int KS>
__global__ __launch_bounds__(NTHREADS, 1) void mla_decode_fwd(FwdParams p) {
  constexpr int KW = NT / KS;          // keys per wave per tile
  constexpr int MT = KW / 16;          // 16-key M tiles per wave per tile
  constexpr int RGS = 16 * (4 / KS);   // rows per work item
  static_assert(2 * TILE_BYTES >= 4 * 16 * OSTRIDE * 4 + 4 * 16 * 8, "staging fits");

  __shared__ __attribute__((aligned(16))) char smem[2 * TILE_BYTES];

  const int n_items = p.header[0];
  const int item_id = blockIdx.x;
  if (item_id >= n_items) return;
  const int32_t* it = p.items + (size_t)item_id * ITEM_INTS;
  const int b = it[0], rg = it[1], t0 = it[2], t1 = it[3], slot = it[4];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int ks = w % KS;
  const int rt = w / KS;

  const int L = min(max(p.seq_lens[b], 0), p.max_keys);
  const int row_local = rt * 16 + c16;
  const int row = rg * RGS + row_local;
  const bool row_ok = row < p.rows;
  int limit = 0;   // keys [t0, limit) are visible to this lane's row
  if (row_ok) {
    int tok = row / p.heads;
    int vis = p.causal ? L - p.s_q + 1 + tok : L;
    limit = min(vis, t1);
  }

  // Q^T operand: lane holds row c16, features 32*s + 8*g .. +7 for s = 0..17.
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

  f32x4_t o[DV / 16];
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max of base-2 scores (row-uniform)
  float l_run = 0.f;         // this lane's share of the running sum

  const size_t row_bytes = KVT == MLA_DTYPE_BF16 ? D * 2 : D;
  const int32_t* bt = p.block_table + (size_t)b * p.max_blocks;
  // A page id outside [0, num_blocks) is a caller error: its keys are read
  // as zeros instead of faulting.
  auto tile_src = [&](int ts, int& n_valid) {
    int page = bt[ts / p.bs];
    if (page < 0 || page >= p.num_blocks) { n_valid = 0; page = 0; }
    return p.kv + ((size_t)page * p.bs + (ts % p.bs)) * row_bytes;
  };

  // Per-lane LDS byte offsets (see lds_off). K operand: key ks*KW + c16,
  // chunk 4*s + g, whose in-row position is (4*(s&1) + g) ^ (c16 & 7).
  int kbase[2];
  kbase[0] = (ks * KW + c16) * 128 + ((g ^ (c16 & 7)) << 4);
  kbase[1] = (ks * KW + c16) * 128 + (((4 + g) ^ (c16 & 7)) << 4);
  // V^T operand by transposed LDS reads: within each 16-lane group, lane
  // s = 4*j + q points at the 8 bytes V[key 4*g + j][dims 16*dt + 4*q .. +3];
  // ds_read_b64_tr_b16 then hands lane c16 the four values V[4*g + 0..3][16*dt + c16].
  // The row's 16-byte chunk is 2*dt + (q >> 1) at in-row position
  // (2*(dt&3) ^ lanex) with lanex = (q >> 1) ^ 4*(g&1) ^ j, so one of four
  // per-lane offsets plus an immediate addresses every read.
  int vt[4];
  {
    const int j = c16 >> 2, q = c16 & 3;
    const int lanex = (q >> 1) ^ ((g & 1) << 2) ^ j;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      vt[c] = (4 * g + j) * 128 + (((2 * c) ^ lanex) << 4) + (q & 1) * 8;
  }

  TileStage<KVT> stage;
  int buf = 0;
  if (t0 < t1) {
    int nv = min(NT, t1 - t0);
    const uint8_t* src = tile_src(t0, nv);
    stage.load(src, nv, tid);
    stage.store(smem, tid);
  }
  __syncthreads();

  for (int ts = t0; ts < t1; ts += NT) {
    const bool has_next = ts + NT < t1;
    if (has_next) {
      int nv = min(NT, t1 - ts - NT);
      const uint8_t* src = tile_src(ts + NT, nv);
      stage.load(src, nv, tid);
    }

    const char* tile = smem + buf * TILE_BYTES;

    // ---- S^T = K Q^T for this wave's MT x 16 keys ----
    // lane reads key kk = ks*KW + 16*mi + c16, chunk 4*s + g: with the swizzle
    // that is kbase[s & 1] + (s >> 1) * 64 rows * 128 B + mi * 16 rows * 128 B.
    f32x4_t sacc[MT];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      sacc[mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const char* src = tile + kbase[s & 1] + (s >> 1) * (NT * 128) + mi * (16 * 128);
        bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(src);
        sacc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[s], sacc[mi], 0, 0, 0);
      }
    }

    // ---- online softmax (base 2), lane = one row, 4*MT keys ----
    float x[MT][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int key = ts + ks * KW + mi * 16 + 4 * g + j;
        float v = sacc[mi][j] * p.scale_log2;
        v = key < limit ? v : -INFINITY;
        x[mi][j] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = wave_max_across_groups(tmax);
    const bool need = tmax > m_run + RESCALE_SLACK;
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
    float pv[MT][4];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float e = m_run == -INFINITY ? 0.f : exp2f(x[mi][j] - m_run);
        pv[mi][j] = e;
        l_run += e;
      }
    }

    // ---- O^T += V^T P^T ----
    if constexpr (MT == 1) {
      // 16 keys: 16x16x16 MFMA, B = P^T (keys 4g..4g+3 of the M tile)
      s16x4_t pb;
      {
        uint32_t p01 = pack_bf16x2(pv[0][0], pv[0][1]);
        uint32_t p23 = pack_bf16x2(pv[0][2], pv[0][3]);
        pb = __builtin_bit_cast(s16x4_t, make_uint2(p01, p23));
      }
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) {
        const s16x4_t a = read_vt(tile + vt[dt & 3] + (dt >> 2) * (NT * 128) + (ks * KW) * 128);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[dt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < MT / 2; ++u) {
        // 32 keys = M tiles 2u and 2u+1; k-slots 0..3 -> keys 4g..4g+3 of the
        // first, k-slots 4..7 -> keys 4g..4g+3 of the second (same in A and B)
        bf16x8_t pb = __builtin_bit_cast(
            bf16x8_t, make_uint4(pack_bf16x2(pv[2 * u][0], pv[2 * u][1]),
                                 pack_bf16x2(pv[2 * u][2], pv[2 * u][3]),
                                 pack_bf16x2(pv[2 * u + 1][0], pv[2 * u + 1][1]),
                                 pack_bf16x2(pv[2 * u + 1][2], pv[2 * u + 1][3])));
#pragma unroll
        for (int dt = 0; dt < DV / 16; ++dt) {
          const char* src = tile + vt[dt & 3] + (dt >> 2) * (NT * 128) + (ks * KW + 32 * u) * 128;
          const s16x4_t a0 = read_vt(src);
          const s16x4_t a1 = read_vt(src + 16 * 128);
          bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, make_uint4(__builtin_bit_cast(uint2, a0).x, __builtin_bit_cast(uint2, a0).y,
                                   __builtin_bit_cast(uint2, a1).x, __builtin_bit_cast(uint2, a1).y));
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[dt], 0, 0, 0);
        }
      }
    }

    if (has_next) stage.store(smem + (buf ^ 1) * TILE_BYTES, tid);
    __syncthreads();
    buf ^= 1;
  }

  merge_and_store<KS>(p, smem, o, m_run, l_run, b, rg, slot);
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
__device__ __forceinline__ void lds_dma16(const char* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(gbase)
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
__global__ __launch_bounds__(NTHREADS, 1) void mla_decode_h16(FwdParams p) {
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
  const int b = it[0], t0 = it[2], t1 = it[3], slot = it[4];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c16 = lane & 15;

  const int L = min(max(p.seq_lens[b], 0), p.max_keys);
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
        lds_dma16(src + (n & 1) * 8 * ROWB + (n >> 1) * 128, dma_lane[0], l0 + n * 1024);
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

  int itn = 0;
  if (w < ntiles) issue(w, wbuf);
  for (int j = w; j < ntiles; j += 4, ++itn) {
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
    const int ts = t0 + KT * j;

    // ---- S^T = K Q^T: MT 16-key M tiles x 16 rows ----
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

    // ---- online softmax (base 2), lane = one row, 4*MT keys ----
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
    const bool need = tmax > m_run + RESCALE_SLACK;
    if (__builtin_amdgcn_ballot_w64(need)) {
      float alpha = 1.f;
      if (need) {
        alpha = exp2f(m_run - tmax);
        m_run = tmax;
      }
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DV / 16; ++d) o[d] *= alpha;
    }
    float pv[MT][4];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float e = m_run == -INFINITY ? 0.f : exp2f(x[mi][jj] - m_run);
        pv[mi][jj] = e;
        l_run += e;
      }

    // ---- O^T += V^T P^T ----
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
  }
  __syncthreads();
  merge_and_store<4>(p, smem, o, m_run, l_run, b, 0, slot);
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

// One workgroup per (sequence, row group); only pairs that were split do work.
// Merge: lse = log2(sum_s 2^lse_s), out = sum_s 2^(lse_s - lse) o_s.
__global__ __launch_bounds__(NTHREADS) void mla_combine_kernel(CombineParams p) {
  const int pair = blockIdx.x;
  if (pair >= p.n_pairs) return;
  const int first = p.pairs[2 * pair];
  const int n = p.pairs[2 * pair + 1];
  if (first < 0 || n <= 1) return;
  const int b = pair / p.nrg, rg = pair % p.nrg;
  const int tpr = NTHREADS / p.rgs;
  const int dpt = DV / tpr;
  const int rr = threadIdx.x / tpr;
  const int d0 = (threadIdx.x % tpr) * dpt;
  const int grow = rg * p.rgs + rr;
  if (grow >= p.rows) return;

  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, p.part_lse[(size_t)(first + s) * p.rgs + rr]);
  float den = 0.f;
  for (int s = 0; s < n; ++s) {
    float ls = p.part_lse[(size_t)(first + s) * p.rgs + rr];
    den += ls == -INFINITY ? 0.f : exp2f(ls - M);
  }
  const bool empty = !(den > 0.f);
  const float inv = empty ? 0.f : 1.f / den;
  const size_t orow = (size_t)b * p.rows + grow;
  for (int d = 0; d < dpt; d += 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < n; ++s) {
      float ls = p.part_lse[(size_t)(first + s) * p.rgs + rr];
      float wgt = ls == -INFINITY ? 0.f : exp2f(ls - M) * inv;
      const float* src = p.part_o + ((size_t)(first + s) * p.rgs + rr) * DV + d0 + d;
      f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(src);
      f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(src + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += wgt * v0[e];
        acc[4 + e] += wgt * v1[e];
      }
    }
    *reinterpret_cast<uint4*>(p.out + orow * DV + d0 + d) =
        make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
  if (p.lse != nullptr && (threadIdx.x % tpr) == 0)
    p.lse[orow] = empty ? -INFINITY : (M + log2f(den)) * LN2;
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
  if (d->num_heads > MLA_MAX_HEADS || s_q > MLA_MAX_SQ) return MLA_ERR_UNSUPPORTED;
  if (d->block_size != 64 && d->block_size != 128) return MLA_ERR_UNSUPPORTED;
  if (d->kv_dtype != MLA_DTYPE_BF16 && d->kv_dtype != MLA_DTYPE_FP8_E4M3FN) return MLA_ERR_UNSUPPORTED;
  if (d->split_keys % NT != 0) return MLA_ERR_INVALID_ARGUMENT;
  long long max_keys = (long long)d->max_blocks_per_seq * d->block_size;
  if (max_keys > (1LL << 30)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

int max_keys_of(const mla_decode_desc_t* d) { return d->max_blocks_per_seq * d->block_size; }

template <int KVT>
void launch_fwd(int ks, dim3 grid, hipStream_t st, const FwdParams& fp) {
  switch (ks) {
    case 4: hipLaunchKernelGGL((mla_decode_fwd<KVT, 4>), grid, dim3(NTHREADS), 0, st, fp); break;
    case 2: hipLaunchKernelGGL((mla_decode_fwd<KVT, 2>), grid, dim3(NTHREADS), 0, st, fp); break;
    default: hipLaunchKernelGGL((mla_decode_fwd<KVT, 1>), grid, dim3(NTHREADS), 0, st, fp); break;
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
  hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, st, pp);
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

mla_status_t launch_fwd_and_combine(const void* q, const void* kv_cache,
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
  if (desc->kv_dtype == MLA_DTYPE_BF16 && rows <= 16)
    hipLaunchKernelGGL(mla_decode_h16<MLA_DTYPE_BF16>, grid, dim3(NTHREADS), 0, hs, fp);
  else if (rows <= 16)
    hipLaunchKernelGGL(mla_decode_h16<MLA_DTYPE_FP8_E4M3FN>, grid, dim3(NTHREADS), 0, hs, fp);
  else if (desc->kv_dtype == MLA_DTYPE_BF16)
    launch_fwd<MLA_DTYPE_BF16>(rc.ks, grid, hs, fp);
  else
    launch_fwd<MLA_DTYPE_FP8_E4M3FN>(rc.ks, grid, hs, fp);
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
  hipLaunchKernelGGL(mla_combine_kernel, dim3(cp.n_pairs), dim3(NTHREADS), 0, hs, cp);
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
  return launch_fwd_and_combine(q, kv_cache, block_table, seq_lens, s_q, softmax_scale, kv_scale,
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
  return launch_fwd_and_combine(q, kv_cache, block_table, seq_lens, s_q, softmax_scale, kv_scale,
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
