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
constexpr int G_TN = 64;                        // output columns per tile
constexpr int G_TK = 32;                        // k per step
constexpr int G_BROW = G_TN * 2 + 8;            // LDS row of the B tile: 136 bytes

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

__global__ __launch_bounds__(G_THREADS) void mla_bgemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) char bt[2][G_TK * G_BROW];
  const int h = blockIdx.z;
  const int t0 = blockIdx.y * G_TM;
  const int n0 = blockIdx.x * G_TN;
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
  // B tile loads: thread -> (k row tid >> 3, 8 columns at 8 * (tid & 7))
  const int bk = tid >> 3, bn = 8 * (tid & 7);
  // B^T operand of column tile nt: lane 4j + q of each 16-lane group supplies
  // columns 16nt + 4q .. +3 of k row 8g + j (+ 4 for the second read)
  const int jj = (lane >> 2) & 3, qq = lane & 3;

  f32x4_t acc[G_TN / 16];
#pragma unroll
  for (int nt = 0; nt < G_TN / 16; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int steps = p.K / G_TK;
  uint4 bnext = *reinterpret_cast<const uint4*>(bmat + (size_t)bk * p.N + bn);
  for (int s = 0; s < steps; ++s) {
    char* buf = bt[s & 1];
    *reinterpret_cast<uint4*>(buf + bk * G_BROW + bn * 2) = bnext;
    if (s + 1 < steps)
      bnext = *reinterpret_cast<const uint4*>(bmat + (size_t)((s + 1) * G_TK + bk) * p.N + bn);
    const uint4 av = t_ok ? *reinterpret_cast<const uint4*>(arow + s * G_TK + 8 * g) : make_uint4(0, 0, 0, 0);
    __syncthreads();   // B tile s in LDS (buffer s & 1 was last read in step s - 2)
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
    for (int nt = 0; nt < G_TN / 16; ++nt) {
      const char* src = buf + (8 * g + jj) * G_BROW + (16 * nt + 4 * qq) * 2;
      const s16x4_t b0 = gemm_read_tr(src);
      const s16x4_t b1 = gemm_read_tr(src + 4 * G_BROW);
      const bf16x8_t bf = __builtin_bit_cast(
          bf16x8_t, make_uint4(__builtin_bit_cast(uint2, b0).x, __builtin_bit_cast(uint2, b0).y,
                               __builtin_bit_cast(uint2, b1).x, __builtin_bit_cast(uint2, b1).y));
      // C^T tile (16 columns x 16 tokens) = B^T (16 x 32) . A^T (32 x 16)
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf, a, acc[nt], 0, 0, 0);
    }
  }
  // acc[nt] lane (c16 = token, g) holds C[t][n0 + 16nt + 4g + j], j = 0..3
  if (t_ok) {
    uint16_t* crow = p.c + ((size_t)t * p.H + h) * p.ldc + n0;
#pragma unroll
    for (int nt = 0; nt < G_TN / 16; ++nt)
      *reinterpret_cast<uint2*>(crow + 16 * nt + 4 * g) =
          make_uint2(pack_bf16x2(acc[nt][0], acc[nt][1]), pack_bf16x2(acc[nt][2], acc[nt][3]));
  }
}

bool al(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

mla_status_t launch_bgemm(const GemmParams& gp, void* stream) {
  if (gp.T == 0) return MLA_OK;
  const dim3 grid(gp.N / G_TN, (gp.T + G_TM - 1) / G_TM, gp.H);
  hipLaunchKernelGGL(mla_bgemm_kernel, grid, dim3(G_THREADS), 0, static_cast<hipStream_t>(stream), gp);
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
  if (tokens < 0 || heads < 1 || heads > MLA_MAX_HEADS || d_v < G_TN) return MLA_ERR_INVALID_ARGUMENT;
  if (d_v % G_TN != 0 || d_v > 4096) return MLA_ERR_UNSUPPORTED;
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
