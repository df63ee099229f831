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
//                          O^T += V^T P^T on MFMA with a base-2 online
//                          softmax; writes the final rows or a split partial
//                          (fp16 normalised o * 2^k, base-2 lse):
//        mla_decode_narrow   <= 16 query rows per sequence (HBM-bound): every
//                            wave streams its own key tiles HBM -> LDS
//        mla_decode_wide     17..64 rows: 64-row items, 16 rows per wave on
//                            16x16x32 MFMA, the waves share the key tiles
//        mla_decode_wide128  > 64 rows: 128-row items on 8 waves of 16 rows
//                            (two waves per SIMD), the waves share the key
//                            tiles
//   3. mla_combine_kernel  merges the partials of split (sequence, row group)
//                          pairs with log-sum-exp weights
#include <algorithm>
#include <cstring>
#include <mutex>

#include "mla_internal.h"

using namespace mla_detail;

namespace {

constexpr int TARGET_ITEMS = 256;    // automatic split: about one work item per CU
constexpr int MIN_CHUNK = 256;       // shortest automatic split chunk (keys)
constexpr int ITEM_OVERHEAD = 96;    // per-item cost of the chunk search, in keys
constexpr int ITEM_OVERHEAD_WIDE128 = 320;
constexpr int HEADER_BYTES = 256;

// ---------------------------------------------------------------------------
// shared host/device planning arithmetic
// ---------------------------------------------------------------------------

// Row grouping: kind 0 = narrow kernel (<= 16 rows), kind 1 = wide kernel
// with 16 rows per wave (64-row items, up to 64 rows), kind 2 = 128-row
// kernel with 8 waves of 16 rows (128-row items, more than 64 rows).
struct RowCfg {
  int kind;
  int rgs;       // query rows per work item
  int nrg;       // row groups per sequence
  int target;    // work items the automatic split aims for
  int overhead;  // per-item cost in key units for the chunk search (below)
};

__host__ __device__ inline RowCfg row_config(int rows) {
  RowCfg c;
  c.kind = rows <= 16 ? 0 : rows <= 64 ? 1 : 2;
  c.rgs = c.kind == 0 ? 16 : c.kind == 1 ? 64 : 128;
  c.nrg = (rows + c.rgs - 1) / c.rgs;
  c.target = TARGET_ITEMS;
  // A 128-row item also loads 147 KB of q and writes a 128 KB fp16 partial
  // that the combine reads back: several times the narrow kernel's overhead.
  c.overhead = c.kind == 2 ? ITEM_OVERHEAD_WIDE128 : ITEM_OVERHEAD;
  return c;
}

__host__ __device__ inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// ceil(a / b) for 0 <= a <= 2^25 and 1 <= b <= 2^25, without an integer
// divide (the planner's candidate search makes many of these): the float
// quotient of two exact operands is within one of the true one, and the two
// corrections make it exact, on the host and on the device alike.
__host__ __device__ inline int ceil_div_small(int a, int b) {
  int q = static_cast<int>(static_cast<float>(a) / static_cast<float>(b));
  if (q * b > a) --q;
  if ((q + 1) * b <= a) ++q;   // q = floor(a / b)
  return q * b == a ? q : q + 1;
}

// Split of one sequence's key range [0, keys) into n chunks of `len` keys
// (len a multiple of the tile); keys == 0 still yields one (empty) chunk.
// Computed in 64-key units (chunk is a multiple of 64, keys <= 2^30), where
// ceil(keys / x) = ceil(ceil(keys / 64) / (x / 64)). With k = ceil(keys / 64)
// and c = chunk / 64: n = ceil(k / c) and len / 64 = l = ceil(k / n), and
// these n chunks of l cover k exactly once more than n - 1 would: l <= c
// (k / n <= c, c an integer), so (n - 1) l <= (n - 1) c < k.
__host__ __device__ inline void seq_split(int keys, int chunk, int* n, int* len) {
  if (keys <= 0) { *n = 1; *len = 0; return; }
  const int k64 = (keys + NT - 1) / NT;
  const int n0 = ceil_div_small(k64, chunk / NT);
  *len = ceil_div_small(k64, n0) * NT;
  *n = n0;
}

// The same arithmetic on the device, in float64: a reciprocal estimate
// refined by one Newton step (relative error far below 2^-40) gives a
// truncated quotient within one of floor(a / b) for a <= 2^25; the remainder
// a - q b is exact in float64 (integers below 2^52) and corrects it. The
// divisor's refined reciprocal is computed once where the divisor repeats.
__device__ __forceinline__ double rcp_refined(double d) {
  const double r = __builtin_amdgcn_rcp(d);
  return __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
}
// floor(a / b) and the remainder, for 0 <= a < 2^31 and 1 <= b <= 2^25
__device__ __forceinline__ int floor_div_dev(int a, double db, double rb, double* rem_out) {
  const double da = a;
  const double q = __builtin_trunc(da * rb);
  const double rem = __builtin_fma(-q, db, da);
  // branch-free correction by -1, 0 or +1
  const double adj = (rem < 0.0 ? -1.0 : 0.0) + (rem >= db ? 1.0 : 0.0);
  *rem_out = __builtin_fma(-adj, db, rem);
  return static_cast<int>(q + adj);
}
__device__ __forceinline__ int ceil_div_dev(int a, double db, double rb) {
  double rem;
  const int q = floor_div_dev(a, db, rb, &rem);
  return rem > 0.0 ? q + 1 : q;
}
// seq_split with the chunk's 64-key count c64 and its refined reciprocal
__device__ __forceinline__ void seq_split_dev(int keys, double c64, double rc, int* n, int* len) {
  if (keys <= 0) { *n = 1; *len = 0; return; }
  const int k64 = (keys + NT - 1) / NT;
  const int n0 = ceil_div_dev(k64, c64, rc);
  const double dn = n0;
  *len = ceil_div_dev(k64, dn, rcp_refined(dn)) * NT;
  *n = n0;
}

__host__ __device__ inline int chunk_from_work(long long work, int forced, int target) {
  if (forced > 0) return forced;
  long long c = (work + target - 1) / target;
  c = (c + NT - 1) / NT * NT;
  if (c < MIN_CHUNK) c = MIN_CHUNK;
  if (c > (1LL << 30)) c = 1LL << 30;
  return static_cast<int>(c);
}

// Automatic chunk length: the decode kernels run one workgroup per CU, so a
// plan is a list schedule of work items on SLOTS workers. For few (sequence,
// row group) pairs the chunk is chosen among CHUNK_CANDIDATES lengths between
// work / (4 * SLOTS) and twice work / SLOTS by an estimate of the makespan in
// key units: every item costs its keys plus an overhead o (prologue, first
// tile latency, partial write); with n items of at most mx keys and wk keys
// in all,
//   n <= SLOTS : mx + o
//   otherwise  : max(mx + o, ceil((wk + n * o) / SLOTS) + (mx + o) / 4).
// The last term is the tail of the schedule: items are issued roughly longest
// first, so the last workers to finish overrun the average by a fraction of
// one item; a simulated list schedule of the skewed 128-head batches gives
// about a fifth of an item. Ties go to the longer chunk (fewer partials).
// With many pairs the split from the average (work / SLOTS) is kept. All integer, so the host mirror
// reproduces the device plan exactly. (A batch of equal lengths keeps the
// average split: every item then has the same length.)
constexpr int SLOTS = 256;
constexpr int CHUNK_CANDIDATES = 32;
constexpr int SEARCH_MAX_PAIRS = 1024;

struct ChunkRange {
  int lo, hi;
  bool search;
};

// Partial slots: a sequence split n >= 2 ways takes n <= 2 (n - 1) slots per
// row group, and n - 1 < (its keys rounded to 64) / chunk, so a plan uses
// fewer than 2 * work / chunk slots. An automatic chunk of at least
// 2 * work / slot_cap therefore keeps every plan within slot_cap slots. With
// the default cap of 8 * SLOTS this is the search's own lower end,
// work / (4 * SLOTS).
constexpr int DEFAULT_SLOT_CAP = 8 * SLOTS;

__host__ __device__ inline int chunk_floor(long long work, int slot_cap) {
  if (slot_cap <= 0) return 1 << 30;   // no slots at all: no splits
  long long c = (2 * work + slot_cap - 1) / slot_cap;
  c = (c + NT - 1) / NT * NT;
  return c > (1LL << 30) ? (1 << 30) : static_cast<int>(c);
}

__host__ __device__ inline ChunkRange chunk_range(long long work, int pairs, bool uniform, int forced,
                                                  int target, int slot_cap) {
  ChunkRange r;
  int c0 = chunk_from_work(work, forced, target);
  const int floor_c = forced == 0 ? chunk_floor(work, slot_cap) : 0;
  if (c0 < floor_c) c0 = floor_c;
  r.search = forced == 0 && pairs < SEARCH_MAX_PAIRS && !uniform;
  r.lo = r.hi = c0;
  if (r.search) {
    r.lo = chunk_from_work(work, 0, 4 * SLOTS);
    if (r.lo < floor_c) r.lo = floor_c;
    r.hi = c0 >= (1 << 29) ? c0 : 2 * c0;
  }
  return r;
}

// Candidate k: lo + k * step with step = ceil((hi - lo) / (candidates - 1))
// rounded up to 64 keys, capped at hi.
__host__ __device__ inline int chunk_step(const ChunkRange& r) {
  return round_up((r.hi - r.lo + CHUNK_CANDIDATES - 2) / (CHUNK_CANDIDATES - 1), NT);
}

__host__ __device__ inline int chunk_candidate(const ChunkRange& r, int step, int k) {
  const long long c = r.lo + (long long)step * k;
  return c < r.hi ? (int)c : r.hi;
}

__host__ __device__ inline unsigned long long plan_cost(unsigned long long n, unsigned long long mx,
                                                        unsigned long long wk, unsigned long long o) {
  if (n <= SLOTS) return mx + o;
  const unsigned long long avg = ((wk + n * o + SLOTS - 1) >> 8) + ((mx + o) >> 2);
  static_assert(SLOTS == 256, "the shift above divides by SLOTS");
  return avg > mx + o ? avg : mx + o;
}

// Upper bound on work items (and partial slots) for a description.
inline long long max_items_bound(int batch, int rows, int max_keys, int forced) {
  RowCfg rc = row_config(rows);
  long long per_seq_cap = (max_keys + NT - 1) / NT;             // chunks are >= 64 keys
  if (forced > 0) per_seq_cap = (max_keys + forced - 1) / forced;
  if (per_seq_cap < 1) per_seq_cap = 1;
  long long cap = (long long)rc.nrg * batch * per_seq_cap;
  if (forced == 0) {
    // the chunk is at least work / (4 * SLOTS): at most 4 * SLOTS items beyond
    // one per (sequence, row group)
    long long auto_cap = 4LL * SLOTS + (long long)rc.nrg * batch;
    long long min_cap = (long long)rc.nrg * batch * ((max_keys + MIN_CHUNK - 1) / MIN_CHUNK);
    if (min_cap < (long long)rc.nrg * batch) min_cap = (long long)rc.nrg * batch;
    if (auto_cap < cap) cap = auto_cap;
    if (min_cap < cap) cap = min_cap;
  }
  return cap;
}

struct WsLayout {
  size_t items, pairs, part_lse, part_scale, part_o, total;
  long long max_items, max_slots;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WsLayout ws_layout(int batch, int s_q, int heads, int max_keys, int forced,
                          int slot_cap = DEFAULT_SLOT_CAP) {
  int rows = s_q * heads;
  RowCfg rc = row_config(rows);
  WsLayout w;
  w.max_items = max_items_bound(batch, rows, max_keys, forced);
  // Partial slots: bounded by the items, and for automatic splits by the
  // planner's slot cap (chunk_floor).
  w.max_slots = w.max_items;
  if (forced == 0 && w.max_slots > slot_cap) w.max_slots = slot_cap;
  size_t off = HEADER_BYTES;
  w.items = off;   off = align256(off + (size_t)w.max_items * ITEM_INTS * 4);
  w.pairs = off;   off = align256(off + (size_t)batch * rc.nrg * 2 * 4);
  w.part_lse = off; off = align256(off + (size_t)w.max_slots * rc.rgs * 4);
  w.part_scale = off; off = align256(off + (size_t)w.max_slots * rc.rgs * 4);
  w.part_o = off;  off = align256(off + (size_t)w.max_slots * rc.rgs * DV * 2);   // fp16
  w.total = off;
  return w;
}

// ---------------------------------------------------------------------------
// planner
// ---------------------------------------------------------------------------

struct PlanParams {
  const int32_t* seq_lens;
  int32_t* header;       // [0] items [1] chunk [2] slots [3] clamp flag
  int32_t* items;        // ITEM_INTS per item
  int32_t* pairs;        // per (b, row group): first slot, number of splits
  int batch, nrg, max_keys, forced_chunk, target, overhead, slot_cap;
  long long max_items, max_slots;
};

constexpr int PLAN_THREADS = 256;
constexpr int PLAN_WAVES = PLAN_THREADS / 64;

// Cross-lane steps on DPP (operands moved between lanes by the VALU, with no
// LDS round trip; the planner is a chain of such steps, so their latency is
// its run time). Controls: quad_perm [1,0,3,2] = 0xB1 and [2,3,0,1] = 0x4E
// (lane ^ 1, lane ^ 2), row_half_mirror 0x141 (lane i <- 7 - i within 8),
// row_mirror 0x140 (i <- 15 - i within 16), row_shr:n 0x110 + n, row_bcast:15
// 0x142 (row r <- lane 15 of row r - 1) and row_bcast:31 0x143 (rows 2, 3 <-
// lane 31). A lane with no source, or in a row the mask leaves out, gets
// `fill`.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_move(int fill, int v) {
  return __builtin_amdgcn_update_dpp(fill, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ long long dpp_move64(long long fill, long long v) {
  const uint64_t f = static_cast<uint64_t>(fill), u = static_cast<uint64_t>(v);
  const uint32_t lo = static_cast<uint32_t>(dpp_move<CTRL, ROWS>(static_cast<int>(f), static_cast<int>(u)));
  const uint32_t hi =
      static_cast<uint32_t>(dpp_move<CTRL, ROWS>(static_cast<int>(f >> 32), static_cast<int>(u >> 32)));
  return static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Inclusive scan over the 64 lanes of a wave: shifts by 1, 2, 4, 8 inside
// each 16-lane row, then the totals of rows 0 and 2 carried into rows 1 and 3,
// then lane 31's into rows 2 and 3. `ident` is op's identity.
template <typename T, typename Op>
__device__ __forceinline__ T wave_scan(T v, T ident, Op op) {
  auto mv = [&](auto ctrl, auto rows, T x) -> T {
    constexpr int C = decltype(ctrl)::value, R = decltype(rows)::value;
    if constexpr (sizeof(T) == 8)
      return dpp_move64<C, R>(ident, x);
    else
      return dpp_move<C, R>(ident, x);
  };
  using std::integral_constant;
  v = op(v, mv(integral_constant<int, 0x111>{}, integral_constant<int, 0xF>{}, v));
  v = op(v, mv(integral_constant<int, 0x112>{}, integral_constant<int, 0xF>{}, v));
  v = op(v, mv(integral_constant<int, 0x114>{}, integral_constant<int, 0xF>{}, v));
  v = op(v, mv(integral_constant<int, 0x118>{}, integral_constant<int, 0xF>{}, v));
  v = op(v, mv(integral_constant<int, 0x142>{}, integral_constant<int, 0xA>{}, v));
  v = op(v, mv(integral_constant<int, 0x143>{}, integral_constant<int, 0xC>{}, v));
  return v;
}
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  return wave_scan(v, 0, [](int a, int b) { return a + b; });
}
// The wave's total (or min / max): lane 63 of the inclusive scan, uniform.
__device__ __forceinline__ int lane63(int v) { return __builtin_amdgcn_readlane(v, 63); }
__device__ __forceinline__ unsigned long long readlane64(unsigned long long u, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(u), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), l);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ long long lane63(long long v) {
  return static_cast<long long>(readlane64(static_cast<unsigned long long>(v), 63));
}

// One workgroup. Thread t owns the contiguous sequences [t*per, (t+1)*per);
// seq_lens are read once into LDS. Block-wide steps: the total work (sum of
// row groups x keys rounded to 64) bounds the chunk length, the candidate
// chunks are costed (few pairs only), then an exclusive scan of per-thread
// item / partial-slot counts places every item. With one sequence per thread
// the items are then written item-parallel (each thread finds an item's
// sequence by a binary search over the scan), otherwise by their owners.
__global__ __launch_bounds__(PLAN_THREADS) void mla_plan_kernel(PlanParams p) {
  extern __shared__ int32_t s_len[];          // batch entries
  __shared__ long long s_work[PLAN_WAVES], s_keys[PLAN_WAVES];
  __shared__ int s_min[PLAN_WAVES], s_max[PLAN_WAVES];
  __shared__ int s_cnt[CHUNK_CANDIDATES], s_mx[CHUNK_CANDIDATES];
  __shared__ int s_long[PLAN_WAVES], s_tail[PLAN_WAVES], s_slots[PLAN_WAVES], s_flag[PLAN_WAVES];
  // one sequence per thread: inclusive scan of long items and first slot per sequence
  __shared__ int s_inc_long[PLAN_THREADS], s_slot0[PLAN_THREADS];
  __shared__ int s_n[PLAN_THREADS], s_chunk_len[PLAN_THREADS];   // the sequence's split
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
  long long work = 0, keys = 0;
  int lmin = INT32_MAX, lmax = 0;
  for (int b = b0; b < b1; ++b) {
    work += (long long)p.nrg * round_up(s_len[b], NT);
    keys += (long long)p.nrg * s_len[b];
    lmin = min(lmin, s_len[b]);
    lmax = max(lmax, s_len[b]);
  }
  // four independent scans per step; lane 63 holds the wave's totals
  auto add64 = [](long long a, long long b) { return a + b; };
  work = lane63(wave_scan(work, 0LL, add64));
  keys = lane63(wave_scan(keys, 0LL, add64));
  lmin = lane63(wave_scan(lmin, INT32_MAX, [](int a, int b) { return min(a, b); }));
  lmax = lane63(wave_scan(lmax, 0, [](int a, int b) { return max(a, b); }));
  const int any_clamped = __any(clamped);
  if (lane == 0) {
    s_work[wv] = work;
    s_keys[wv] = keys;
    s_min[wv] = lmin;
    s_max[wv] = lmax;
    s_flag[wv] = any_clamped;
  }
  __syncthreads();
  long long total = 0, total_keys = 0;
  int flag = 0;
  lmin = INT32_MAX;
  lmax = 0;
#pragma unroll
  for (int i = 0; i < PLAN_WAVES; ++i) {
    total += s_work[i];
    total_keys += s_keys[i];
    lmin = min(lmin, s_min[i]);
    lmax = max(lmax, s_max[i]);
    flag |= s_flag[i];
  }
  const ChunkRange cr = chunk_range(total, p.batch * p.nrg, lmin == lmax, p.forced_chunk, p.target,
                                    p.slot_cap);
  int chunk = cr.lo;
  if (cr.search) {
    // items and longest item for every candidate chunk (8 threads per
    // candidate, all candidates at once), then the cheapest
    constexpr int TPC = PLAN_THREADS / CHUNK_CANDIDATES;
    static_assert(TPC <= 64 && (TPC & (TPC - 1)) == 0, "the xor steps below stay inside a wave");
    const int step = chunk_step(cr);
    {
      const int k = tid / TPC, sub = tid % TPC;
      const int c = chunk_candidate(cr, step, k);
      // four sequences per iteration: independent division chains overlap
      const double c64 = c / NT, rc = rcp_refined(c64);
      int cnt = 0, mx = 0;
      int b = sub;
      for (; b + 3 * TPC < p.batch; b += 4 * TPC) {
        int n[4], len[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) seq_split_dev(s_len[b + u * TPC], c64, rc, &n[u], &len[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          cnt += n[u];
          mx = max(mx, min(len[u], s_len[b + u * TPC]));
        }
      }
      for (; b < p.batch; b += TPC) {
        int n, len;
        seq_split_dev(s_len[b], c64, rc, &n, &len);
        cnt += n;
        mx = max(mx, min(len, s_len[b]));
      }
      // sums over the 8 lanes of a candidate: lane ^ 1, lane ^ 2, then the
      // other quad of the half row
      static_assert(TPC == 8, "the three DPP steps below cover 8 lanes");
      cnt += dpp_move<0xB1, 0xF>(0, cnt);
      mx = max(mx, dpp_move<0xB1, 0xF>(0, mx));
      cnt += dpp_move<0x4E, 0xF>(0, cnt);
      mx = max(mx, dpp_move<0x4E, 0xF>(0, mx));
      cnt += dpp_move<0x141, 0xF>(0, cnt);
      mx = max(mx, dpp_move<0x141, 0xF>(0, mx));
      if (sub == 0) {
        s_cnt[k] = cnt;
        s_mx[k] = mx;
      }
    }
    __syncthreads();
    // argmin over the candidates (ties: the larger k) as the minimum of
    // cost * 32 + (31 - k): a search runs for fewer than SEARCH_MAX_PAIRS
    // pairs, so the work is below 2^40 keys and every cost below 2^34
    static_assert(CHUNK_CANDIDATES == 32, "five bits of candidate index");
    unsigned long long key = ~0ull;
    if (lane < CHUNK_CANDIDATES)
      key = (plan_cost((unsigned long long)s_cnt[lane] * p.nrg, s_mx[lane], total_keys, p.overhead) << 5) |
            static_cast<unsigned long long>(CHUNK_CANDIDATES - 1 - lane);
    auto kmin = [](unsigned long long a, long long b) {
      const unsigned long long ub = static_cast<unsigned long long>(b);
      return a < ub ? a : ub;
    };
    key = kmin(key, dpp_move64<0xB1, 0xF>(-1LL, static_cast<long long>(key)));
    key = kmin(key, dpp_move64<0x4E, 0xF>(-1LL, static_cast<long long>(key)));
    key = kmin(key, dpp_move64<0x141, 0xF>(-1LL, static_cast<long long>(key)));
    key = kmin(key, dpp_move64<0x140, 0xF>(-1LL, static_cast<long long>(key)));
    // lanes 0 and 16 hold the minima of candidates 0..15 and 16..31
    const unsigned long long k0 = readlane64(key, 0), k1 = readlane64(key, 16);
    const unsigned long long best = k0 < k1 ? k0 : k1;
    chunk = chunk_candidate(cr, step, CHUNK_CANDIDATES - 1 - static_cast<int>(best & 31));
  }

  const double chunk64 = chunk / NT, rchunk = rcp_refined(chunk64);
  int my_long = 0, my_tail = 0, my_slots = 0;
  for (int b = b0; b < b1; ++b) {
    int n, len;
    seq_split_dev(s_len[b], chunk64, rchunk, &n, &len);
    if (per == 1) {
      s_n[tid] = n;
      s_chunk_len[tid] = len;
    }
    my_long += p.nrg * (n - 1);
    my_tail += p.nrg;
    if (n > 1) my_slots += p.nrg * n;
  }
  const int inc_long = wave_inclusive_scan(my_long);
  const int inc_tail = wave_inclusive_scan(my_tail);
  const int inc_slots = wave_inclusive_scan(my_slots);
  if (lane == 63) {
    s_long[wv] = inc_long;
    s_tail[wv] = inc_tail;
    s_slots[wv] = inc_slots;
  }
  __syncthreads();
  int litem = inc_long - my_long, titem = inc_tail - my_tail, slot = inc_slots - my_slots;
  int tot_long = 0, tot_tail = 0, tot_slots = 0;
#pragma unroll
  for (int i = 0; i < PLAN_WAVES; ++i) {
    if (i < wv) {
      litem += s_long[i];
      titem += s_tail[i];
      slot += s_slots[i];
    }
    tot_long += s_long[i];
    tot_tail += s_tail[i];
    tot_slots += s_slots[i];
  }
  titem += tot_long;
  const int tot_items = tot_long + tot_tail;
  // Cannot happen within the workspace bounds; if it did, no item runs and
  // the header says so (bit 1 of the flag word).
  const bool overflow = tot_items > p.max_items || tot_slots > p.max_slots;
  // Pair (b, rg) owns the partial slots slot_b + rg * n .. + n - 1. Items go
  // longest first: every chunk but a sequence's last (all of full length)
  // before the last chunks, chunk-major within each class, so the row groups
  // of one chunk stay consecutive (side by side on one XCD, sharing its L2
  // for the cache rows).
  auto write_item = [&](int item, int b, int rg, int s, int n, int len, int L, int slot_b) {
    if (item < p.max_items) {
      int4* it = reinterpret_cast<int4*>(p.items + (size_t)item * ITEM_INTS);
      it[0] = make_int4(b, rg, s * len, min(L, (s + 1) * len));
      it[1] = make_int4(n > 1 ? slot_b + rg * n + s : -1, 0, 0, 0);
    }
  };
  if (per == 1) {
    // thread b owns sequence b: publish its long-item scan and first slot,
    // then write items and pairs spread over all threads
    const int me_long = overflow ? 0 : my_long;
    const int inc = litem + me_long;   // exclusive start + own count
    s_inc_long[tid] = tid < p.batch ? inc : INT32_MAX;
    s_slot0[tid] = slot;
    __syncthreads();
    const int n_long = overflow ? 0 : tot_long;
    const double dnrg = p.nrg, rnrg = rcp_refined(dnrg);
    for (int i = tid; i < n_long; i += PLAN_THREADS) {
      // the sequence of long item i: the first b with inclusive scan > i
      int lo = 0, hi = p.batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_inc_long[mid] > i) hi = mid; else lo = mid + 1;
      }
      const int b = lo, L = s_len[b];
      const int n = s_n[b], len = s_chunk_len[b];
      const int local = i - (s_inc_long[b] - p.nrg * (n - 1));
      double rg;
      const int s = floor_div_dev(local, dnrg, rnrg, &rg);
      write_item(i, b, static_cast<int>(rg), s, n, len, L, s_slot0[b]);
    }
    const int n_tail = p.batch * p.nrg;
    for (int i = tid; i < n_tail; i += PLAN_THREADS) {
      // last chunks: nrg per sequence, in sequence order; also the pair entry
      double drg;
      const int b = floor_div_dev(i, dnrg, rnrg, &drg), rg = static_cast<int>(drg), L = s_len[b];
      int n = s_n[b];
      const int len = s_chunk_len[b];
      if (overflow) n = 1;
      write_item(n_long + i, b, rg, n - 1, n, len, L, s_slot0[b]);
      p.pairs[2 * i] = n > 1 ? s_slot0[b] + rg * n : -1;
      p.pairs[2 * i + 1] = n;
    }
  } else {
    for (int b = b0; b < b1; ++b) {
      const int L = s_len[b];
      int n, len;
      seq_split_dev(L, chunk64, rchunk, &n, &len);
      if (overflow) n = 1;
      for (int rg = 0; rg < p.nrg; ++rg) {
        p.pairs[2 * (b * p.nrg + rg)] = n > 1 ? slot + rg * n : -1;
        p.pairs[2 * (b * p.nrg + rg) + 1] = n;
      }
      for (int s = 0; s < n; ++s)
        for (int rg = 0; rg < p.nrg; ++rg) {
          int& item = s < n - 1 ? litem : titem;
          write_item(item, b, rg, s, n, len, L, slot);
          ++item;
        }
      if (n > 1) slot += p.nrg * n;
    }
  }
  if (tid == 0) {
    p.header[0] = overflow ? 0 : tot_items;
    p.header[1] = chunk;
    p.header[2] = tot_slots;
    p.header[3] = (flag ? FLAG_SEQ_LEN_CLAMPED : 0) | (overflow ? FLAG_PLAN_OVERFLOW : 0);
  }
}

// ---------------------------------------------------------------------------
// combine kernel
// ---------------------------------------------------------------------------

struct CombineParams {
  const int32_t* pairs;
  const _Float16* part_o;
  const float* part_lse;
  const int32_t* part_scale;
  uint16_t* out;
  float* lse;
  int32_t* flags;   // header word 3: FLAG_BAD_ITEM for a pair whose slots do not fit
  int rows, rgs, nrg, n_pairs, max_slots;
};

// Grid (pair, chunk): thread (row, 8-dim slice) of one (sequence, row group)
// pair; only pairs that were split do work. Merge of the pair's n partials:
// lse = log2(sum_s 2^lse_s), out = sum_s 2^(lse_s - lse) o_s, where the
// partial rows hold fp16 values of o_s * 2^k_s with a per-row exponent k_s.
constexpr int COMBINE_SLICES = DV / 8;   // 64 threads per row
static_assert(COMBINE_SLICES == 64, "one wave per row: the combine reads the row index as wave-uniform");

__global__ __launch_bounds__(NTHREADS) void mla_combine_kernel(CombineParams p) {
  const int pair = blockIdx.x;
  const int first = p.pairs[2 * pair];
  const int n = p.pairs[2 * pair + 1];
  if (first < 0 || n <= 1) return;
  if ((long long)first + n > p.max_slots) {   // a stale plan (see item_in_range)
    flag_bad_item(p.flags);
    return;
  }
  // one wave per row: the row index is wave-uniform, so the per-split lse
  // and exponent loads are scalar (C3 combine 9.8 -> 9.4 us, C4 16.2 -> 15.9)
  const int rr = __builtin_amdgcn_readfirstlane(blockIdx.y * (NTHREADS / COMBINE_SLICES) +
                                                (int)(threadIdx.x / COMBINE_SLICES));
  const int d0 = (threadIdx.x % COMBINE_SLICES) * 8;
  const int b = pair / p.nrg, rg = pair % p.nrg;
  const int grow = rg * p.rgs + rr;
  if (rr >= p.rgs || grow >= p.rows) return;

  // Splits are taken four at a time with all their loads issued together (one
  // memory round trip per four splits), merged with a running max: the sum
  // is rescaled by 2^(M_old - M_new) whenever a group raises the max.
  constexpr int CB = 4;
  const float* lse_s = p.part_lse + (size_t)first * p.rgs + rr;
  const int32_t* k_s = p.part_scale + (size_t)first * p.rgs + rr;
  const size_t elem = ((size_t)first * p.rgs + rr) * DV + d0;   // element offset of split 0
  const size_t sstride = (size_t)p.rgs * DV;
  float M = -INFINITY, den = 0.f;
  f32x4_t acc0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  for (int s0 = 0; s0 < n; s0 += CB) {
    float l[CB];
    int ks[CB];
    f32x4_t a[CB], c[CB];
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      if (s0 + i < n) {
        l[i] = lse_s[(size_t)(s0 + i) * p.rgs];
        ks[i] = k_s[(size_t)(s0 + i) * p.rgs];
        const f16x8_t h = *reinterpret_cast<const f16x8_t*>(p.part_o + elem + (s0 + i) * sstride);
        a[i] = f32x4_t{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
        c[i] = f32x4_t{(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
      } else {
        l[i] = -INFINITY;
        ks[i] = 0;
        a[i] = c[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    float Mc = M;
#pragma unroll
    for (int i = 0; i < CB; ++i) Mc = fmaxf(Mc, l[i]);
    const float sc = M == -INFINITY ? 0.f : exp2f(M - Mc);   // the sum so far is 0 while M = -inf
    den *= sc;
    acc0 *= sc;
    acc1 *= sc;
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const float w = l[i] == -INFINITY ? 0.f : exp2f(l[i] - Mc);
      den += w;
      const float wo = __builtin_ldexpf(w, -ks[i]);   // undo the row's 2^k
      acc0 += wo * a[i];
      acc1 += wo * c[i];
    }
    M = Mc;
  }
  float acc[8] = {acc0[0], acc0[1], acc0[2], acc0[3], acc1[0], acc1[1], acc1[2], acc1[3]};
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
  // the plan's item and slot counts are int32 and size the decode grid
  if (max_items_bound(d->batch, s_q * d->num_heads, static_cast<int>(max_keys), d->split_keys) > (1LL << 30))
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

int max_keys_of(const mla_decode_desc_t* d) { return d->max_blocks_per_seq * d->block_size; }

void launch_decode(int kv_dtype, int kind, dim3 grid, hipStream_t st, const FwdParams& fp) {
  if (kind == 0)
    launch_narrow(kv_dtype, grid, st, fp);
  else if (kind == 1)
    launch_wide(kv_dtype, grid, st, fp);
  else
    launch_wide128(kv_dtype, grid, st, fp);
}

mla_status_t launch_plan(const int32_t* seq_lens, int32_t s_q, const mla_decode_desc_t* desc,
                         void* workspace, const WsLayout& ws, hipStream_t st,
                         int slot_cap = DEFAULT_SLOT_CAP) {
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
  pp.overhead = rc.overhead;
  pp.max_keys = max_keys_of(desc);
  pp.forced_chunk = desc->split_keys;
  pp.max_items = ws.max_items;
  pp.max_slots = ws.max_slots;
  pp.slot_cap = slot_cap;
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

// Host-only checks of the decode arguments other than the workspace.
mla_status_t check_args(const void* q, const void* kv_cache, const int32_t* block_table,
                        const int32_t* seq_lens, int32_t s_q, float softmax_scale,
                        float kv_scale, const void* out, const float* lse,
                        const mla_decode_desc_t* desc) {
  mla_status_t st = check_desc(s_q, desc);
  if (st != MLA_OK) return st;
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f) ||
      !(std::isfinite(kv_scale) && kv_scale > 0.f))
    return MLA_ERR_INVALID_ARGUMENT;
  if (q == nullptr || kv_cache == nullptr || block_table == nullptr || seq_lens == nullptr ||
      out == nullptr)
    return MLA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || (lse != nullptr && !aligned(lse, 4)))
    return MLA_ERR_INVALID_ARGUMENT;
  return MLA_OK;
}

mla_status_t check_call(const void* q, const void* kv_cache, const int32_t* block_table,
                        const int32_t* seq_lens, int32_t s_q, float softmax_scale,
                        float kv_scale, const void* out, const float* lse,
                        const mla_decode_desc_t* desc, const void* workspace,
                        size_t workspace_bytes, WsLayout* ws) {
  mla_status_t st = check_args(q, kv_cache, block_table, seq_lens, s_q, softmax_scale, kv_scale,
                               out, lse, desc);
  if (st != MLA_OK) return st;
  if (workspace == nullptr || !aligned(workspace, 256)) return MLA_ERR_INVALID_ARGUMENT;
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
  fp.flags = reinterpret_cast<int32_t*>(base) + 3;
  fp.items = reinterpret_cast<const int32_t*>(base + ws.items);
  fp.part_o = reinterpret_cast<_Float16*>(base + ws.part_o);
  fp.part_lse = reinterpret_cast<float*>(base + ws.part_lse);
  fp.part_scale = reinterpret_cast<int32_t*>(base + ws.part_scale);
  fp.heads = desc->num_heads;
  fp.s_q = s_q;
  fp.rows = rows;
  fp.bs = desc->block_size;
  fp.max_blocks = desc->max_blocks_per_seq;
  fp.max_keys = max_keys_of(desc);
  fp.causal = desc->causal;
  fp.num_blocks = desc->num_blocks;
  fp.batch = desc->batch;
  fp.max_items = static_cast<int>(ws.max_items);
  fp.max_slots = static_cast<int>(ws.max_slots);
  fp.scale_log2 = softmax_scale * kv_scale * LOG2E;
  fp.out_scale = kv_scale;
  // a multiple of 8 workgroups: the wide kernel deals items out per XCD
  dim3 grid(static_cast<unsigned>((ws.max_items + 7) / 8 * 8));
  launch_decode(desc->kv_dtype, rc.kind, grid, hs, fp);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  if (!combine) return MLA_OK;

  CombineParams cp;
  cp.pairs = reinterpret_cast<const int32_t*>(base + ws.pairs);
  cp.part_o = fp.part_o;
  cp.part_lse = fp.part_lse;
  cp.part_scale = fp.part_scale;
  cp.out = fp.out;
  cp.lse = lse;
  cp.rows = rows;
  cp.rgs = rc.rgs;
  cp.nrg = rc.nrg;
  cp.n_pairs = desc->batch * rc.nrg;
  cp.flags = fp.flags;
  cp.max_slots = fp.max_slots;
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

mla_status_t mla_decode_with_plan(const void* q, const void* kv_cache, const int32_t* block_table,
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
                                true);
}

int32_t mla_plan_host(const int32_t* seq_lens_host, int32_t s_q, const mla_decode_desc_t* desc,
                      int32_t* items, int32_t max_items, int32_t* rows_per_item,
                      int32_t* chunk_keys) {
  if (check_desc(s_q, desc) != MLA_OK || (desc->batch > 0 && seq_lens_host == nullptr))
    return -1;
  RowCfg rc = row_config(s_q * desc->num_heads);
  const int max_keys = max_keys_of(desc);
  long long work = 0, keys = 0;
  int lmin = INT32_MAX, lmax = 0;
  for (int b = 0; b < desc->batch; ++b) {
    int L = std::min(std::max(seq_lens_host[b], 0), max_keys);
    work += (long long)rc.nrg * round_up(L, NT);
    keys += (long long)rc.nrg * L;
    lmin = std::min(lmin, L);
    lmax = std::max(lmax, L);
  }
  const ChunkRange cr = chunk_range(work, desc->batch * rc.nrg, lmin == lmax, desc->split_keys, rc.target,
                                    DEFAULT_SLOT_CAP);
  int chunk = cr.lo;
  if (cr.search) {
    const int step = chunk_step(cr);
    unsigned long long best = ~0ull;
    for (int k = 0; k < CHUNK_CANDIDATES; ++k) {
      const int c = chunk_candidate(cr, step, k);
      long long n = 0;
      int mx = 0;
      for (int b = 0; b < desc->batch; ++b) {
        int L = std::min(std::max(seq_lens_host[b], 0), max_keys);
        int nb, len;
        seq_split(L, c, &nb, &len);
        n += nb;
        mx = std::max(mx, std::min(len, L));
      }
      const unsigned long long cost = plan_cost((unsigned long long)n * rc.nrg, mx, keys, rc.overhead);
      if (cost <= best) {
        best = cost;
        chunk = c;
      }
    }
  }
  if (rows_per_item) *rows_per_item = rc.rgs;
  if (chunk_keys) *chunk_keys = chunk;
  // two passes, as on the device: every chunk but the last of each sequence,
  // then the last chunks; slots per (b, row group) pair as on the device
  int item = 0;
  for (int pass = 0; pass < 2; ++pass) {
    int slot = 0;
    for (int b = 0; b < desc->batch; ++b) {
      int L = std::min(std::max(seq_lens_host[b], 0), max_keys);
      int n, len;
      seq_split(L, chunk, &n, &len);
      for (int s = pass == 0 ? 0 : n - 1; s < (pass == 0 ? n - 1 : n); ++s)
        for (int rg = 0; rg < rc.nrg; ++rg) {
          if (item >= max_items) return -1;
          if (items) {
            int32_t* it = items + (size_t)item * ITEM_INTS;
            it[0] = b; it[1] = rg; it[2] = s * len; it[3] = std::min(L, (s + 1) * len);
            it[4] = n > 1 ? slot + rg * n + s : -1; it[5] = 0; it[6] = 0; it[7] = 0;
          }
          ++item;
        }
      if (n > 1) slot += rc.nrg * n;
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

// ---------------------------------------------------------------------------
// decode without a caller workspace: plan, work items and split partials live
// in a fixed device array of this library
// ---------------------------------------------------------------------------

namespace {

// One copy per GPU, held from the library's load until the process ends. In
// host code `scratch` names a host-side stand-in, never the device memory:
// kernels get the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The device address of `scratch` on the current device (looked up once per
// device), or nullptr if the lookup fails.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// A workspace layout that fits the scratch array: the regular one when it
// fits (the plan is then the same as mla_decode's), else automatic splits
// with as many partial slots as fit. Returns false if nothing fits.
bool scratch_layout(int32_t s_q, const mla_decode_desc_t* desc, WsLayout* ws, int* slot_cap) {
  const int mk = max_keys_of(desc);
  *slot_cap = DEFAULT_SLOT_CAP;
  *ws = ws_layout(desc->batch, s_q, desc->num_heads, mk, desc->split_keys);
  if (ws->total <= MLA_NOALLOC_SCRATCH_BYTES) return true;
  if (desc->split_keys != 0) return false;
  const WsLayout none = ws_layout(desc->batch, s_q, desc->num_heads, mk, 0, 0);
  if (none.total > MLA_NOALLOC_SCRATCH_BYTES) return false;
  const size_t per_slot = (size_t)row_config(s_q * desc->num_heads).rgs * (4 + 4 + DV * 2);
  int cap = static_cast<int>((MLA_NOALLOC_SCRATCH_BYTES - none.total) / per_slot);
  // the three partial regions are each rounded up to 256 bytes
  while (cap > 0 && ws_layout(desc->batch, s_q, desc->num_heads, mk, 0, cap).total > MLA_NOALLOC_SCRATCH_BYTES)
    --cap;
  *slot_cap = cap;
  *ws = ws_layout(desc->batch, s_q, desc->num_heads, mk, 0, cap);
  return ws->total <= MLA_NOALLOC_SCRATCH_BYTES;
}

}  // namespace

extern "C" {

size_t mla_decode_noalloc_scratch_bytes(void) { return MLA_NOALLOC_SCRATCH_BYTES; }

mla_status_t mla_decode_noalloc(const void* q, const void* kv_cache, const int32_t* block_table,
                                const int32_t* seq_lens, int32_t s_q, float softmax_scale,
                                float kv_scale, void* out, float* lse,
                                const mla_decode_desc_t* desc, void* stream) {
  mla_status_t st = check_args(q, kv_cache, block_table, seq_lens, s_q, softmax_scale, kv_scale,
                               out, lse, desc);
  if (st != MLA_OK) return st;
  WsLayout ws;
  int slot_cap = DEFAULT_SLOT_CAP;
  if (!scratch_layout(s_q, desc, &ws, &slot_cap)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (desc->batch == 0) return MLA_OK;
  void* base = scratch_on_current_device();
  if (base == nullptr) return MLA_ERR_HIP;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  st = launch_plan(seq_lens, s_q, desc, base, ws, hs, slot_cap);
  if (st != MLA_OK) return st;
  return launch_decode_kernel(q, kv_cache, block_table, seq_lens, s_q, softmax_scale, kv_scale, out,
                              lse, desc, base, ws, hs, true);
}

}  // extern "C"
