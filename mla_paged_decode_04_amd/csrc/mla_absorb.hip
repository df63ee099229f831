// The absorbed projections around the decode MQA ("[WIP][Attention] FlashAttn
// MLA", description: the decode step of MLA is computed as MQA). Reading used
// (the pages give no shapes for it): per head h,
//   q[t, h, 0:512]   = q_nope[t, h, :] . W_UK[h]     (d_nope -> 512 latent)
//   q[t, h, 512:576] = q_pe[t, h, :]                 (the rotary part, copied)
//   out[t, h, :]     = o[t, h, 0:512] . W_UV[h]      (512 latent -> d_v)
// with bf16 inputs and weights, fp32 accumulation and a bf16 result. Both are
// batched GEMMs C[h] = A[h] . B[h] on 16x16x32 bf16 MFMA tiles.
#include "mla_internal.h"

using namespace mla_detail;

namespace {

constexpr int G_THREADS = 256;                  // 4 waves
constexpr int G_TM = 64;                        // tokens per tile (16 per wave)
constexpr int G_TK = 32;                        // k per step

// Weight-stationary shape of absorb_out with d_v other than 128 (column
// slice, A read-ahead in k-steps, token tiles per workgroup); tuning knobs.
#ifndef ABSO_TN
#define ABSO_TN 64
#endif
#ifndef ABSO_AHEAD
#define ABSO_AHEAD 16
#endif
#ifndef ABSO_TPW
#define ABSO_TPW 32
#endif

// Ring kernels: workgroups per launch (about), LDS ring slots of absorb_q
// and absorb_out.
#ifndef RSQ_WGS
#define RSQ_WGS 256
#endif
#ifndef RSQ_DEPTH
#define RSQ_DEPTH 8
#endif
#ifndef RSO_DEPTH
#define RSO_DEPTH 5
#endif

struct GemmParams {
  const uint16_t* a;       // A(t, h, k) = a[(t * H + h) * lda + k]
  const uint16_t* b;       // B(h, k, n) = b[(h * K + k) * N + n]
  uint16_t* c;             // C(t, h, n) = c[(t * H + h) * ldc + n]
  const uint16_t* pe;      // absorb_q only: q_pe(t, h, 0:64) copied to C(t, h, 512:576)
  int T, H, K, N, lda, ldc;
};

// ds_read_b64_tr_b16 (see the decode kernels for the lane mapping).
__device__ __forceinline__ s16x4_t gemm_read_tr(const char* p) {
  typedef __attribute__((address_space(3))) s16x4_t lds_t;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_t*)(p));
}

// One workgroup: 64 tokens x TN output columns of one head. The B tile of
// every k-step (32 x TN) is staged in LDS (double-buffered, one barrier per
// step); the lane's A fragment comes from global memory one step ahead. With
// TN covering a whole output row (512 for absorb_q, d_v for absorb_out), the
// C tile is staged in LDS at the end and every row leaves as one contiguous
// run (the output is the larger part of the traffic).
template <int TN>
__global__ __launch_bounds__(G_THREADS) void mla_bgemm_kernel(GemmParams p) {
  constexpr int BROW = TN * 2 + 8;              // LDS row of the B tile (bytes)
  constexpr int CROW = TN * 2 + 16;             // LDS row of the staged C tile (bytes)
  constexpr int B_BYTES = 2 * G_TK * BROW;
  constexpr int C_BYTES = G_TM * CROW;
  __shared__ __attribute__((aligned(16))) char lds[B_BYTES > C_BYTES ? B_BYTES : C_BYTES];
  const int h = blockIdx.z;
  const int t0 = blockIdx.y * G_TM;
  const int n0 = blockIdx.x * TN;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;

  // the rotary part of q rides along with the first column tile
  if (p.pe != nullptr && blockIdx.x == 0) {
    for (int i = tid; i < G_TM * 8; i += G_THREADS) {
      const int t = t0 + (i >> 3), c = i & 7;
      if (t < p.T)
        *reinterpret_cast<uint4*>(p.c + ((size_t)t * p.H + h) * p.ldc + 512 + 8 * c) =
            *reinterpret_cast<const uint4*>(p.pe + ((size_t)t * p.H + h) * 64 + 8 * c);
    }
  }

  const int t = t0 + 16 * w + c16;                       // this lane's A row
  const bool t_ok = t < p.T;
  const uint16_t* arow = p.a + ((size_t)(t_ok ? t : 0) * p.H + h) * p.lda;
  const uint16_t* bmat = p.b + (size_t)h * p.K * p.N + n0;
  // B tile loads: 16-byte chunk i of the step's 32 x TN tile is k row
  // i / (TN / 8), columns 8 (i % (TN / 8)); each thread takes chunks tid + 256 m
  constexpr int BCH = G_TK * TN / 8 / G_THREADS;        // chunks per thread
  // B^T operand of column tile nt: lane 4j + q of each 16-lane group supplies
  // columns 16nt + 4q .. +3 of k row 8g + j (+ 4 for the second read)
  const int jj = (lane >> 2) & 3, qq = lane & 3;

  f32x4_t acc[TN / 16];
#pragma unroll
  for (int nt = 0; nt < TN / 16; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int steps = p.K / G_TK;
  uint4 bnext[BCH];
  auto load_b = [&](int s) {
#pragma unroll
    for (int m = 0; m < BCH; ++m) {
      const int i = tid + G_THREADS * m;
      bnext[m] = *reinterpret_cast<const uint4*>(bmat + (size_t)(s * G_TK + i / (TN / 8)) * p.N + 8 * (i % (TN / 8)));
    }
  };
  auto load_a = [&](int s) {
    return t_ok ? *reinterpret_cast<const uint4*>(arow + s * G_TK + 8 * g) : make_uint4(0, 0, 0, 0);
  };
  load_b(0);
  uint4 anext = load_a(0);
  for (int s = 0; s < steps; ++s) {
    char* buf = lds + (s & 1) * G_TK * BROW;
#pragma unroll
    for (int m = 0; m < BCH; ++m) {
      const int i = tid + G_THREADS * m;
      *reinterpret_cast<uint4*>(buf + (i / (TN / 8)) * BROW + (i % (TN / 8)) * 16) = bnext[m];
    }
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, anext);
    if (s + 1 < steps) {
      load_b(s + 1);
      anext = load_a(s + 1);
    }
    __syncthreads();   // B tile s in LDS (buffer s & 1 was last read in step s - 2)
#pragma unroll
    for (int nt = 0; nt < TN / 16; ++nt) {
      const char* src = buf + (8 * g + jj) * BROW + (16 * nt + 4 * qq) * 2;
      const s16x4_t b0 = gemm_read_tr(src);
      const s16x4_t b1 = gemm_read_tr(src + 4 * BROW);
      const bf16x8_t bf = __builtin_bit_cast(
          bf16x8_t, make_uint4(__builtin_bit_cast(uint2, b0).x, __builtin_bit_cast(uint2, b0).y,
                               __builtin_bit_cast(uint2, b1).x, __builtin_bit_cast(uint2, b1).y));
      // C^T tile (16 columns x 16 tokens) = B^T (16 x 32) . A^T (32 x 16)
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf, a, acc[nt], 0, 0, 0);
    }
  }
  // acc[nt] lane (c16 = token, g) holds C[t][n0 + 16nt + 4g + j], j = 0..3:
  // stage the 64 x TN tile as bf16, then write whole row runs
  __syncthreads();   // every wave is done with the B buffers
  {
    char* crow = lds + (16 * w + c16) * CROW;
#pragma unroll
    for (int nt = 0; nt < TN / 16; ++nt)
      *reinterpret_cast<uint2*>(crow + (16 * nt + 4 * g) * 2) =
          make_uint2(pack_bf16x2(acc[nt][0], acc[nt][1]), pack_bf16x2(acc[nt][2], acc[nt][3]));
  }
  __syncthreads();
  constexpr int CCH = TN / 8;                            // 16-byte chunks per row
  for (int i = tid; i < G_TM * CCH; i += G_THREADS) {
    const int r = i / CCH, c = i % CCH;
    const int tt = t0 + r;
    if (tt < p.T)
      *reinterpret_cast<uint4*>(p.c + ((size_t)tt * p.H + h) * p.ldc + n0 + 8 * c) =
          *reinterpret_cast<const uint4*>(lds + r * CROW + c * 16);
  }
}

// Weight-stationary variant for many tokens: the workgroup keeps its head's
// K x TN slice of B in LDS for the whole launch and runs TPW token tiles of 64
// through it, so B is read once per workgroup instead of once per 64 tokens.
// A fragments are read from global memory AH k-steps ahead (a register ring
// whose slot for flat k-step f is f % AH; AH divides the k-steps per tile),
// which keeps enough reads in flight with one workgroup per CU. No barrier is
// needed inside a tile: B does not change.
//
// The grid is one-dimensional and XCD-aware: workgroups are dealt to the 8
// XCDs in turn, so the column slices of one (token group, head) get ids 8
// apart. They then run side by side on one XCD, and the A rows they all read
// come from HBM once, into that XCD's L2, instead of once per slice.
template <int TN, int KMAX, int WS_AHEAD, int WS_TPW>   // WS_TPW: token tiles per workgroup
__global__ __launch_bounds__(G_THREADS) void mla_bgemm_ws_kernel(GemmParams p) {
  constexpr int BROW = TN * 2 + 8;
  constexpr int CROW = TN * 2 + 16;
  __shared__ __attribute__((aligned(16))) char bsm[KMAX * BROW];
  __shared__ __attribute__((aligned(16))) char csm[G_TM * CROW];
  const int ns = p.N / TN;                                   // column slices
  const int groups = ((p.T + G_TM - 1) / G_TM + WS_TPW - 1) / WS_TPW;
  const int j = blockIdx.x >> 3;
  const int pair = (j / ns) * 8 + (blockIdx.x & 7);         // (token group, head)
  if (pair >= groups * p.H) return;
  const int h = pair % p.H;
  const int gy = pair / p.H;
  const int n0 = (j % ns) * TN;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int jj = (lane >> 2) & 3, qq = lane & 3;
  const int K = p.K;
  const int steps = K / G_TK;

  // B slice: K rows x TN columns, 16-byte chunks spread over all threads
  {
    const uint16_t* bmat = p.b + (size_t)h * K * p.N + n0;
    for (int i = tid; i < K * (TN / 8); i += G_THREADS) {
      const int r = i / (TN / 8), c = i % (TN / 8);
      *reinterpret_cast<uint4*>(bsm + r * BROW + c * 16) =
          *reinterpret_cast<const uint4*>(bmat + (size_t)r * p.N + 8 * c);
    }
  }
  __syncthreads();

  const int tile0 = gy * WS_TPW;
  const int ntile = min(WS_TPW, (p.T + G_TM - 1) / G_TM - tile0);
  // the flat k-step sequence of this workgroup: tile u, step s -> u * steps + s
  const int total = ntile * steps;
  auto load_a = [&](int f) {
    const int u = f / steps, s = f - u * steps;
    const int t = (tile0 + u) * G_TM + 16 * w + c16;
    if (t >= p.T) return make_uint4(0, 0, 0, 0);
    return *reinterpret_cast<const uint4*>(p.a + ((size_t)t * p.H + h) * p.lda + s * G_TK + 8 * g);
  };
  uint4 ring[WS_AHEAD];
#pragma unroll
  for (int i = 0; i < WS_AHEAD; ++i) ring[i] = i < total ? load_a(i) : make_uint4(0, 0, 0, 0);

  for (int u = 0; u < ntile; ++u) {
    const int t0 = (tile0 + u) * G_TM;
    if (p.pe != nullptr && n0 == 0) {   // the rotary part of q
      for (int i = tid; i < G_TM * 8; i += G_THREADS) {
        const int t = t0 + (i >> 3), c = i & 7;
        if (t < p.T)
          *reinterpret_cast<uint4*>(p.c + ((size_t)t * p.H + h) * p.ldc + 512 + 8 * c) =
              *reinterpret_cast<const uint4*>(p.pe + ((size_t)t * p.H + h) * 64 + 8 * c);
      }
    }
    f32x4_t acc[TN / 16];
#pragma unroll
    for (int nt = 0; nt < TN / 16; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < steps; s += WS_AHEAD) {
#pragma unroll
      for (int i = 0; i < WS_AHEAD; ++i) {
        {
          const int f = u * steps + s + i;
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ring[i]);
          if (f + WS_AHEAD < total) ring[i] = load_a(f + WS_AHEAD);
          const char* bk = bsm + (s + i) * G_TK * BROW;
#pragma unroll
          for (int nt = 0; nt < TN / 16; ++nt) {
            const char* src = bk + (8 * g + jj) * BROW + (16 * nt + 4 * qq) * 2;
            const s16x4_t b0 = gemm_read_tr(src);
            const s16x4_t b1 = gemm_read_tr(src + 4 * BROW);
            const bf16x8_t bf = __builtin_bit_cast(
                bf16x8_t, make_uint4(__builtin_bit_cast(uint2, b0).x, __builtin_bit_cast(uint2, b0).y,
                                     __builtin_bit_cast(uint2, b1).x, __builtin_bit_cast(uint2, b1).y));
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf, a, acc[nt], 0, 0, 0);
          }
        }
      }
    }
    // stage the 64 x TN tile as bf16, then write whole row runs
    {
      char* crow = csm + (16 * w + c16) * CROW;
#pragma unroll
      for (int nt = 0; nt < TN / 16; ++nt)
        *reinterpret_cast<uint2*>(crow + (16 * nt + 4 * g) * 2) =
            make_uint2(pack_bf16x2(acc[nt][0], acc[nt][1]), pack_bf16x2(acc[nt][2], acc[nt][3]));
    }
    __syncthreads();
    constexpr int CCH = TN / 8;
    for (int i = tid; i < G_TM * CCH; i += G_THREADS) {
      const int r = i / CCH, c = i % CCH;
      const int tt = t0 + r;
      if (tt < p.T)
        *reinterpret_cast<uint4*>(p.c + ((size_t)tt * p.H + h) * p.ldc + n0 + 8 * c) =
            *reinterpret_cast<const uint4*>(csm + r * CROW + c * 16);
    }
    __syncthreads();   // csm is rewritten by the next tile
  }
}

// Byte range [base, base + bytes) as a buffer resource (gfx9 descriptor,
// 32-bit data format, no stride, no swizzle; bytes < 2^31: the ring kernels
// build one per 16-row tile). A buffer store whose offset lies outside the
// range is dropped, so every lane of a wave issues the same stores and rows
// past the last token need no branch (a store under a branch, or in a loop
// of unknown length, leaves the compiler's count of memory operations in
// flight inexact, and its next wait then drains all of them).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t byte_range(const void* base, long long bytes) {
  const int n = bytes <= 0 ? 0 : static_cast<int>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
constexpr uint32_t OUT_OF_RANGE = 0x80000000u;   // an offset past every range built here
// AUX: cache-policy bits of the store; 2 = nt (non-temporal, streaming).
template <int AUX = 0>
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, uint4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, off, 0, AUX);
}
constexpr int ST_NT = 2;

// Poll an LDS counter until it reaches `target`, at most 2^22 times (with
// s_sleep 1 between polls, about a tenth of a second): the caller then goes
// on regardless. The compiler keeps the LDS accesses after the call below
// the poll.
__device__ __forceinline__ void lds_await(int* c, int target) {
  for (int i = 0; i < (1 << 22); ++i) {
    if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}

// absorb_q with d_nope = 128: q[t, h, 0:512] = q_nope[t, h, :] . W_UK[h] and
// q[t, h, 512:576] = q_pe[t, h, :]. One workgroup per (token range, head),
// 9 waves in two roles:
// - a loader wave copies each 16-token tile of q_nope (4 KB) and q_pe (2 KB)
//   HBM -> LDS (global_load_lds_dwordx4, non-temporal) into a ring of D tile
//   slots, D - 1 tiles ahead. It issues nothing else, so its vmcnt waits
//   cover its own copies only.
// - 8 compute waves each keep a 128 x 64 column slice of W_UK[h] in VGPRs as
//   MFMA fragments (loaded once through a per-wave LDS staging area and the
//   transposed LDS reads), read the tile's A fragments from the ring, and
//   write results straight from the accumulators: two v_permlane16_swap per
//   register pair turn the 4-column pieces of lanes g and g + 1 into 16-byte
//   runs, and one DPP row rotate lets each store cover 8 whole rows of the
//   wave's 128-byte slice. Wave w also copies q_pe rows 2w and 2w + 1 of the
//   tile. These waves issue stores only and never wait for memory.
// Vector memory operations of a wave retire in issue order; with loads and
// stores in one wave, every load would also wait for the write
// acknowledgements of the stores before it, and under a write-heavy stream
// those arrive late. Slots change hands through two LDS counters instead of a
// barrier per tile (which would start every wave's stores at the same moment):
// the loader publishes how many tiles have landed, and each compute wave
// counts its completions of a slot, which the loader awaits before refilling
// it. Compute waves may thus drift up to D - 1 tiles apart. Every wait on a
// counter gives up after a fixed number of polls, so a broken handshake ends
// the kernel with wrong output instead of a hang. Rows past the last token:
// the copies read the last valid row again and the buffer stores drop them.
constexpr int RS_TM = 16;             // tokens per tile
constexpr int RS_NW = 8;              // compute waves
constexpr int RS_THREADS = (RS_NW + 1) * 64;
constexpr int RS_ATILE = RS_TM * 256; // q_nope tile bytes (d_nope = 128)
constexpr int RS_SLOT = RS_ATILE + RS_TM * 128;
constexpr int RS_NDMA = RS_SLOT / 1024;   // loader transfers per tile
template <int D>   // ring slots
__global__ __launch_bounds__(RS_THREADS) void mla_absorb_q_rs_kernel(GemmParams p, int tpw) {
  constexpr int K = 128, N = 512, NW = RS_NW;
  constexpr int NTW = N / 16 / NW;               // 16-column blocks per wave
  constexpr int WCOL = 16 * NTW;                 // columns per wave
  constexpr int SROW = WCOL * 2 + 8;             // staging row of B (bytes)
  constexpr int KS = K / G_TK;                   // k-steps
  constexpr int STG = NW * G_TK * SROW;
  static_assert(NTW == 4 && RS_TM == 2 * NW, "the output swaps assume 64 columns and 2 q_pe rows per wave");
  static_assert(D >= 2 && RS_NDMA * (D - 1) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char lds[STG + D * RS_SLOT];
  // cnt[0]: tiles landed in the ring; cnt[1 + s]: compute-wave completions of slot s
  __shared__ int cnt[1 + D];
  char* const ring = lds + STG;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int h = blockIdx.x % p.H;
  const int row0 = (blockIdx.x / p.H) * tpw * RS_TM;
  if (row0 >= p.T) return;
  const int rows = min(tpw * RS_TM, p.T - row0);
  const int ntile = (rows + RS_TM - 1) / RS_TM;
  const long long ra_row = (long long)p.H * p.lda * 2;   // bytes between consecutive tokens
  const long long rc_row = (long long)p.H * p.ldc * 2;
  const long long rp_row = (long long)p.H * 64 * 2;
  const char* a0 = reinterpret_cast<const char*>(p.a + ((size_t)row0 * p.H + h) * p.lda);
  const char* p0 = reinterpret_cast<const char*>(p.pe + ((size_t)row0 * p.H + h) * 64);
  if (tid <= D) cnt[tid] = 0;
  __syncthreads();   // the only barrier: the counters start at zero

  if (w == NW) {
    // ---- loader. Slot layout: q_nope row r (256 B) at r * 256 with its
    // 16-byte chunk c at position c ^ r (the compute waves' 16-byte reads
    // are then free of bank conflicts); q_pe row r at RS_ATILE + r * 128.
    // Transfer j, lane l fills slot bytes 1024 j + 16 l.
    const uint32_t ring_lds = lds_addr(ring);
    auto issue = [&](int u) {
      const uint32_t sl = ring_lds + (u % D) * RS_SLOT;
#pragma unroll
      for (int j = 0; j < RS_NDMA; ++j) {
        const int pos = 64 * j + lane;                  // 16-byte position in the slot
        if (j < RS_ATILE / 1024) {
          const int r = pos >> 4, c = (pos & 15) ^ r;
          const int t = min(u * RS_TM + r, rows - 1);
          lds_dma16_nt(a0, (uint32_t)(t * ra_row) + 16 * c, sl + 1024 * j);
        } else {
          const int q = pos - RS_ATILE / 16, r = q >> 3, c = q & 7;
          const int t = min(u * RS_TM + r, rows - 1);
          lds_dma16_nt(p0, (uint32_t)(t * rp_row) + 16 * c, sl + 1024 * j);
        }
      }
    };
    for (int u = 0; u < D - 1; ++u) issue(u);
    for (int u = 0; u < ntile; ++u) {
      wait_vmcnt<RS_NDMA * (D - 2)>();   // tile u has landed (tiles u+1 .. u+D-2 may be in flight)
      __hip_atomic_store(&cnt[0], u + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (u > 0) {   // slot (u - 1) % D is refilled once every compute wave is done with tile u - 1
        const int need = NW * ((u - 1) / D + 1);
        lds_await(&cnt[1 + (u - 1) % D], need);
      }
      issue(u + D - 1);
    }
    wait_vmcnt<0>();   // no copy may land after the workgroup's LDS is released
    return;
  }

  // ---- compute waves: B slice of this wave into registers, frag[nt][s] ----
  const int jj = (lane >> 2) & 3, qq = lane & 3;
  bf16x8_t frag[NTW][KS];
  {
    char* st = lds + w * G_TK * SROW;
    const uint16_t* bw = p.b + (size_t)h * K * N + w * WCOL;
    constexpr int CPR = WCOL / 8;                  // 16-byte chunks per staged row
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int i = lane; i < G_TK * CPR; i += 64) {
        const int r = i / CPR, c = i % CPR;
        *reinterpret_cast<uint4*>(st + r * SROW + c * 16) =
            *reinterpret_cast<const uint4*>(bw + (size_t)(s * G_TK + r) * N + 8 * c);
      }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const char* src = st + (8 * g + jj) * SROW + (16 * nt + 4 * qq) * 2;
        const s16x4_t b0 = gemm_read_tr(src);
        const s16x4_t b1 = gemm_read_tr(src + 4 * SROW);
        frag[nt][s] = __builtin_bit_cast(
            bf16x8_t, make_uint4(__builtin_bit_cast(uint2, b0).x, __builtin_bit_cast(uint2, b0).y,
                                 __builtin_bit_cast(uint2, b1).x, __builtin_bit_cast(uint2, b1).y));
      }
    }
  }

  const char* c0 = reinterpret_cast<const char*>(p.c + ((size_t)row0 * p.H + h) * p.ldc);
  // lane (c16, g) stores into rows c16 & 7 and (c16 & 7) + 8 of each tile
  const uint32_t c_col = 2 * w * WCOL + whole_row_col(c16, g);
  const uint32_t c_off_lo = (uint32_t)((c16 & 7) * rc_row) + c_col;
  const uint32_t c_off_hi = (uint32_t)(((c16 & 7) + 8) * rc_row) + c_col;
  const int prow = 2 * w + ((lane >> 3) & 1);      // q_pe: lanes 0..15 copy rows 2w, 2w + 1
  const uint32_t pc_off = lane < 16 ? (uint32_t)(prow * rc_row) + 2 * N + 16 * (lane & 7) : OUT_OF_RANGE;
  const int pe_lds = RS_ATILE + prow * 128 + 16 * (lane & 7);
  for (int u = 0; u < ntile; ++u) {
    lds_await(&cnt[0], u + 1);   // slot u % D holds tile u
    const char* sl = ring + (u % D) * RS_SLOT;
    f32x4_t acc[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8_t a = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const uint4*>(sl + c16 * 256 + (((4 * s + g) ^ c16) << 4)));
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag[nt][s], a, acc[nt], 0, 0, 0);
    }
    const uint4 pe = *reinterpret_cast<const uint4*>(sl + pe_lds);
    // LDS operations of a wave execute in order: the count follows the reads
    asm volatile("" ::: "memory");
    if (lane == 0) __hip_atomic_fetch_add(&cnt[1 + u % D], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    // acc[nt] lane (c16 = token, g) holds C[c16][w * WCOL + 16nt + 4g + j];
    // each of the two stores covers 8 whole rows of the wave's 128-byte
    // slice (whole_row_runs). Non-temporal: the 604 MB of q at 4096 tokens x
    // 128 heads would otherwise sit dirty in the caches and be written back
    // during the next kernel (absorb_q then absorb_out: 303 -> 290 us).
    uint32_t pk[NTW][2];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      pk[nt][0] = pack_bf16x2(acc[nt][0], acc[nt][1]);
      pk[nt][1] = pack_bf16x2(acc[nt][2], acc[nt][3]);
    }
    uint4 rows_lo, rows_hi;
    whole_row_runs(pk, c16, rows_lo, rows_hi);
    const int left = min(RS_TM, rows - u * RS_TM);   // valid rows of tile u
    const rsrc_t rc = byte_range(c0 + (long long)u * RS_TM * rc_row, (long long)(left - 1) * rc_row + 2 * (N + 64));
    buf_store16<ST_NT>(rc, c_off_lo, rows_lo);
    buf_store16<ST_NT>(rc, c_off_hi, rows_hi);
    buf_store16<ST_NT>(rc, pc_off, pe);
  }
}

// absorb_out with 512 latent columns and d_v = 128: out[t, h, :] =
// o[t, h, :] . W_UV[h]. The same two roles as absorb_q, 9 waves:
// - the loader copies each 16-token tile of o (16 rows of 1 KB, one transfer
//   per row) HBM -> LDS into a ring of D slots, D - 1 tiles ahead;
// - 8 compute waves: wave w keeps the 512 x 32 column slice 32 * (w % 4) of
//   W_UV[h] in VGPRs (two 16-column blocks x 16 k-steps of fragments) and
//   takes the tiles u with u % 2 == w / 4, so each tile is read from LDS by
//   4 waves and every SIMD runs two waves. After two v_permlane16_swap per
//   register a lane holds a 16-byte run, and a wave writes its 64 bytes of
//   the tile's 16 rows in one store.
// Slot layout: token row r at r * 1024 with its 16-byte chunk c at position
// (c & 48) | ((c ^ r) & 15), which keeps the compute waves' 16-byte reads
// free of bank conflicts. The handshake is the one of absorb_q (LDS counters,
// bounded polls).
constexpr int RO_NW = 8;
constexpr int RO_THREADS = (RO_NW + 1) * 64;
constexpr int RO_SLOT = RS_TM * 1024;
template <int D>
__global__ __launch_bounds__(RO_THREADS) void mla_absorb_out_rs_kernel(GemmParams p, int tpw) {
  constexpr int K = 512, N = 128, NTW = 2, WCOL = 32, KS = K / G_TK, NCG = N / WCOL;
  constexpr int SROW = WCOL * 2 + 8;             // staging row of B (bytes)
  constexpr int STG = RO_NW * G_TK * SROW;
  constexpr int NDMA = RS_TM;                    // one 1 KB row per transfer
  static_assert(NCG * 2 == RO_NW && D >= 2 && NDMA * (D - 2) < 64, "shape");
  __shared__ __attribute__((aligned(16))) char lds[STG + D * RO_SLOT];
  __shared__ int cnt[1 + D];   // [0]: tiles landed; [1 + s]: compute-wave completions of slot s
  char* const ring = lds + STG;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int h = blockIdx.x % p.H;
  const int row0 = (blockIdx.x / p.H) * tpw * RS_TM;
  if (row0 >= p.T) return;
  const int rows = min(tpw * RS_TM, p.T - row0);
  const int ntile = (rows + RS_TM - 1) / RS_TM;
  const long long ra_row = (long long)p.H * p.lda * 2;
  const long long rc_row = (long long)p.H * p.ldc * 2;
  const char* a0 = reinterpret_cast<const char*>(p.a + ((size_t)row0 * p.H + h) * p.lda);
  if (tid <= D) cnt[tid] = 0;
  __syncthreads();   // the only barrier: the counters start at zero

  if (w == RO_NW) {   // ---- loader
    const uint32_t ring_lds = lds_addr(ring);
    const int chunk = (lane & 48);
    auto issue = [&](int u) {
      const uint32_t sl = ring_lds + (u % D) * RO_SLOT;
#pragma unroll
      for (int r = 0; r < NDMA; ++r) {
        const int c = chunk | ((lane ^ r) & 15);
        const int t = min(u * RS_TM + r, rows - 1);
        lds_dma16_nt(a0, (uint32_t)(t * ra_row) + 16 * c, sl + 1024 * r);
      }
    };
    for (int u = 0; u < D - 1; ++u) issue(u);
    for (int u = 0; u < ntile; ++u) {
      wait_vmcnt<NDMA * (D - 2)>();   // tile u has landed
      __hip_atomic_store(&cnt[0], u + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (u > 0) lds_await(&cnt[1 + (u - 1) % D], 4 * ((u - 1) / D + 1));   // 4 waves read each tile
      issue(u + D - 1);
    }
    wait_vmcnt<0>();   // no copy may land after the workgroup's LDS is released
    return;
  }

  // ---- compute waves: column group cg, tiles of parity tp
  const int cg = w % NCG, tp = w / NCG;
  const int jj = (lane >> 2) & 3, qq = lane & 3;
  bf16x8_t frag[NTW][KS];
  {
    char* st = lds + w * G_TK * SROW;
    const uint16_t* bw = p.b + (size_t)h * K * N + cg * WCOL;
    constexpr int CPR = WCOL / 8;                  // 16-byte chunks per staged row
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int i = lane; i < G_TK * CPR; i += 64) {
        const int r = i / CPR, c = i % CPR;
        *reinterpret_cast<uint4*>(st + r * SROW + c * 16) =
            *reinterpret_cast<const uint4*>(bw + (size_t)(s * G_TK + r) * N + 8 * c);
      }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const char* src = st + (8 * g + jj) * SROW + (16 * nt + 4 * qq) * 2;
        const s16x4_t b0 = gemm_read_tr(src);
        const s16x4_t b1 = gemm_read_tr(src + 4 * SROW);
        frag[nt][s] = __builtin_bit_cast(
            bf16x8_t, make_uint4(__builtin_bit_cast(uint2, b0).x, __builtin_bit_cast(uint2, b0).y,
                                 __builtin_bit_cast(uint2, b1).x, __builtin_bit_cast(uint2, b1).y));
      }
    }
  }
  const char* c0 = reinterpret_cast<const char*>(p.c + ((size_t)row0 * p.H + h) * p.ldc);
  const uint32_t c_off = (uint32_t)(c16 * rc_row) + 2 * (cg * WCOL + (g & 1) * 16 + (g >> 1) * 8);
  for (int u = tp; u < ntile; u += 2) {
    lds_await(&cnt[0], u + 1);   // slot u % D holds tile u
    const char* sl = ring + (u % D) * RO_SLOT + c16 * 1024;
    f32x4_t acc[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int c = 4 * s + g;
      const bf16x8_t a = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const uint4*>(sl + (((c & 48) | ((c ^ c16) & 15)) << 4)));
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag[nt][s], a, acc[nt], 0, 0, 0);
    }
    // LDS operations of a wave execute in order: the count follows the reads
    asm volatile("" ::: "memory");
    if (lane == 0) __hip_atomic_fetch_add(&cnt[1 + u % D], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    uint32_t pk[NTW][2];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      pk[nt][0] = pack_bf16x2(acc[nt][0], acc[nt][1]);
      pk[nt][1] = pack_bf16x2(acc[nt][2], acc[nt][3]);
    }
#pragma unroll
    for (int d = 0; d < 2; ++d) {   // lane g: columns {0, 16, 8, 24}[g] .. + 7 of the wave's 32
      const auto sw = __builtin_amdgcn_permlane16_swap(pk[0][d], pk[1][d], false, false);
      pk[0][d] = sw[0];
      pk[1][d] = sw[1];
    }
    const int left = min(RS_TM, rows - u * RS_TM);
    const rsrc_t rc = byte_range(c0 + (long long)u * RS_TM * rc_row, (long long)(left - 1) * rc_row + 2 * N);
    buf_store16(rc, c_off, make_uint4(pk[0][0], pk[0][1], pk[1][0], pk[1][1]));
  }
}

bool al(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

mla_status_t launch_bgemm(const GemmParams& gp, void* stream) {
  if (gp.T == 0) return MLA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int tiles = (gp.T + G_TM - 1) / G_TM;     // 64-token tiles
  const int tiles16 = (gp.T + RS_TM - 1) / RS_TM;  // 16-token tiles
  // Ring kernels (at least 16 tiles of 16 tokens; absorb_q with d_nope = 128,
  // absorb_out with d_v = 128): about RSQ_WGS workgroups in all (one per CU
  // at 256), each over a contiguous range of at most 4096 tokens of one head.
  const bool q_ring = gp.K == 128 && gp.N == 512 && gp.pe != nullptr;
  const bool out_ring = gp.K == 512 && gp.N == 128 && gp.pe == nullptr;
  if (tiles16 >= 16 && (q_ring || out_ring)) {
    const int groups = std::max(1, RSQ_WGS / gp.H);
    const int tpw = std::min(256, (tiles16 + groups - 1) / groups);
    const unsigned n = (unsigned)(((tiles16 + tpw - 1) / tpw) * gp.H);
    if (q_ring)
      hipLaunchKernelGGL((mla_absorb_q_rs_kernel<RSQ_DEPTH>), dim3(n), dim3(RS_THREADS), 0, st, gp, tpw);
    else
      hipLaunchKernelGGL((mla_absorb_out_rs_kernel<RSO_DEPTH>), dim3(n), dim3(RO_THREADS), 0, st, gp, tpw);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  }
  // absorb_out with another d_v and many tokens: weight-stationary, on a
  // one-dimensional XCD-aware grid of 8 x slices x ceil(pairs / 8)
  // workgroups. Narrow column slices keep the LDS per workgroup small enough
  // for two or more workgroups per CU.
  if (gp.K == 512 && gp.N % ABSO_TN == 0 && tiles >= 64) {
    const long long pairs = (long long)((tiles + ABSO_TPW - 1) / ABSO_TPW) * gp.H;
    const dim3 grid(static_cast<unsigned>(8LL * (gp.N / ABSO_TN) * ((pairs + 7) / 8)));
    hipLaunchKernelGGL((mla_bgemm_ws_kernel<ABSO_TN, 512, ABSO_AHEAD, ABSO_TPW>), grid, dim3(G_THREADS), 0, st, gp);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  }
  // everything else (few tokens, other shapes): streaming. absorb_q (N = 512)
  // takes whole 512-column rows per tile when there are enough tiles;
  // otherwise 64-column tiles keep more workgroups in flight over the long K
  const int tn = gp.N == 512 && tiles * gp.H >= 512 ? 512 : 64;
  const dim3 grid(gp.N / tn, tiles, gp.H);
  switch (tn) {
    case 512: hipLaunchKernelGGL(mla_bgemm_kernel<512>, grid, dim3(G_THREADS), 0, st, gp); break;
    default: hipLaunchKernelGGL(mla_bgemm_kernel<64>, grid, dim3(G_THREADS), 0, st, gp); break;
  }
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

extern "C" mla_status_t mla_absorb_q(const void* q_nope, const void* q_pe, const void* w_uk, void* q_out,
                                     int32_t tokens, int32_t heads, int32_t d_nope, void* stream) {
  if (tokens < 0 || heads < 1 || heads > MLA_MAX_HEADS || d_nope < G_TK) return MLA_ERR_INVALID_ARGUMENT;
  if (d_nope % G_TK != 0 || d_nope > 4096) return MLA_ERR_UNSUPPORTED;
  if (tokens == 0) return MLA_OK;
  if (q_nope == nullptr || q_pe == nullptr || w_uk == nullptr || q_out == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (!al(q_nope, 16) || !al(q_pe, 16) || !al(w_uk, 16) || !al(q_out, 16)) return MLA_ERR_INVALID_ARGUMENT;
  GemmParams gp;
  gp.a = static_cast<const uint16_t*>(q_nope);
  gp.b = static_cast<const uint16_t*>(w_uk);
  gp.c = static_cast<uint16_t*>(q_out);
  gp.pe = static_cast<const uint16_t*>(q_pe);
  gp.T = tokens;
  gp.H = heads;
  gp.K = d_nope;
  gp.N = DV;
  gp.lda = d_nope;
  gp.ldc = D;
  return launch_bgemm(gp, stream);
}

extern "C" mla_status_t mla_absorb_out(const void* o, const void* w_uv, void* out, int32_t tokens,
                                       int32_t heads, int32_t d_v, void* stream) {
  if (tokens < 0 || heads < 1 || heads > MLA_MAX_HEADS || d_v < 64) return MLA_ERR_INVALID_ARGUMENT;
  if (d_v % 64 != 0 || d_v > 4096) return MLA_ERR_UNSUPPORTED;
  if (tokens == 0) return MLA_OK;
  if (o == nullptr || w_uv == nullptr || out == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (!al(o, 16) || !al(w_uv, 16) || !al(out, 16)) return MLA_ERR_INVALID_ARGUMENT;
  GemmParams gp;
  gp.a = static_cast<const uint16_t*>(o);
  gp.b = static_cast<const uint16_t*>(w_uv);
  gp.c = static_cast<uint16_t*>(out);
  gp.pe = nullptr;
  gp.T = tokens;
  gp.H = heads;
  gp.K = DV;
  gp.N = d_v;
  gp.lda = DV;
  gp.ldc = d_v;
  return launch_bgemm(gp, stream);
}
