// Writing new latent rows into the paged cache (the step before decode):
// "[Attention] Blackwell FP8 MLA support with CUTLASS_MLA backend", Purpose and
// Test Plan -- the latent cache is kept in torch.float8_e4m3fn. A new bf16 row x
// goes to slot s (page s / bs, row s % bs) as y = x / kv_scale (float32,
// correctly rounded), encoded as OCP e4m3fn (clamped to +-448, nearest, ties to
// even mantissa) or as bf16 (nearest, ties to even). Decoding multiplies by
// kv_scale again.
#include "mla_internal.h"

using namespace mla_detail;

namespace {

constexpr int APPEND_THREADS = 256;
constexpr int CHUNKS = D / 8;   // 72 chunks of 8 values per row

// float32 -> OCP e4m3fn code: saturate to 448, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float y) {
  const uint32_t u = __builtin_bit_cast(uint32_t, y);
  const uint32_t sign = (u >> 24) & 0x80u;
  float a = fabsf(y);
  if (a != a) return 0x7Fu | sign;                 // NaN
  a = fminf(a, 448.f);                               // saturate (infinities too)
  if (a < 0.015625f) {                               // below 2^-6: steps of 2^-9
    const float q = __builtin_rintf(a * 512.f);      // exact scaling, ties to even
    return sign | static_cast<uint32_t>(q);          // 0..8 (8 encodes 2^-6)
  }
  const uint32_t b = __builtin_bit_cast(uint32_t, a);
  const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);   // keep 3 mantissa bits, ties to even
  const uint32_t e = (r >> 23) - 120u;                   // rebias 127 -> 7: 1..15
  return sign | (e << 3) | ((r >> 20) & 7u);
}

// Four float32 values -> four OCP e4m3fn codes in one dword, by gfx950's
// v_cvt_scalef32_pk_fp8_f32 (scale 1), two values per instruction. The
// instruction rounds to nearest even but turns magnitudes beyond 448 into NaN,
// so the inputs are clamped to +-448 first; clamped, it gives the same code as
// f32_to_e4m3fn above for every non-NaN float32 (all 2^32 inputs compared on
// MI355X). NaN inputs take f32_to_e4m3fn.
__device__ __forceinline__ uint32_t f32x4_to_e4m3fn(float y0, float y1, float y2, float y3) {
  if (__builtin_expect((y0 != y0) | (y1 != y1) | (y2 != y2) | (y3 != y3), 0))
    return f32_to_e4m3fn(y0) | (f32_to_e4m3fn(y1) << 8) | (f32_to_e4m3fn(y2) << 16) | (f32_to_e4m3fn(y3) << 24);
  auto clamp = [](float y) { return __builtin_fminf(__builtin_fmaxf(y, -448.f), 448.f); };
  s16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2_t{0, 0}, clamp(y0), clamp(y1), 1.0f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, clamp(y2), clamp(y3), 1.0f, true);
  return __builtin_bit_cast(uint32_t, r);
}

struct AppendParams {
  const uint16_t* rows;
  const int32_t* slots;
  uint8_t* kv;
  long long n_slots;   // num_blocks * block_size
  int n_tokens;
  double inv_scale;    // 1 / kv_scale, rounded once to double on the host
};

// y = x / kv_scale, correctly rounded to float32, as one double product
// rounded to float: for a bf16 x (8 significant bits) and a float32 scale the
// exact quotient is never a float32 rounding midpoint (that would need x to
// have 25 or more significant bits), and its distance to one is at least
// about 2^-49 relative, against at most about 2^-52 of error in
// double(x) * double(1 / kv_scale). So rounding the product gives the same
// float as the division (also for overflow, zero, infinities and NaN).
template <int KVT>
__global__ __launch_bounds__(APPEND_THREADS) void mla_kv_append_kernel(AppendParams p) {
  const long long gid = (long long)blockIdx.x * APPEND_THREADS + threadIdx.x;
  if (gid >= (long long)p.n_tokens * CHUNKS) return;
  const int n = static_cast<int>(gid / CHUNKS);
  const int c = static_cast<int>(gid - (long long)n * CHUNKS);
  const long long slot = p.slots[n];
  if (slot < 0 || slot >= p.n_slots) return;        // padding or out of range: no write
  const uint4 raw = *reinterpret_cast<const uint4*>(p.rows + (size_t)n * D + 8 * c);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float y[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    y[2 * k] = static_cast<float>(static_cast<double>(__builtin_bit_cast(float, w[k] << 16)) * p.inv_scale);
    y[2 * k + 1] = static_cast<float>(static_cast<double>(__builtin_bit_cast(float, w[k] & 0xFFFF0000u)) * p.inv_scale);
  }
  if constexpr (KVT == MLA_DTYPE_FP8_E4M3FN) {
    *reinterpret_cast<uint2*>(p.kv + (size_t)slot * D + 8 * c) =
        make_uint2(f32x4_to_e4m3fn(y[0], y[1], y[2], y[3]), f32x4_to_e4m3fn(y[4], y[5], y[6], y[7]));
  } else {
    *reinterpret_cast<uint4*>(p.kv + ((size_t)slot * D + 8 * c) * 2) =
        make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                   pack_bf16x2(y[6], y[7]));
  }
}

bool is_aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

}  // namespace

extern "C" mla_status_t mla_kv_append(const void* rows, const int32_t* slot_mapping, int32_t n_tokens,
                                      float kv_scale, void* kv_cache, int32_t num_blocks,
                                      int32_t block_size, int32_t kv_dtype, void* stream) {
  if (n_tokens < 0 || num_blocks < 1) return MLA_ERR_INVALID_ARGUMENT;
  if (block_size != 64 && block_size != 128) return MLA_ERR_UNSUPPORTED;
  if (kv_dtype != MLA_DTYPE_BF16 && kv_dtype != MLA_DTYPE_FP8_E4M3FN) return MLA_ERR_UNSUPPORTED;
  if (!(std::isfinite(kv_scale) && kv_scale > 0.f)) return MLA_ERR_INVALID_ARGUMENT;
  if (n_tokens == 0) return MLA_OK;
  if (rows == nullptr || slot_mapping == nullptr || kv_cache == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (!is_aligned(rows, 16) || !is_aligned(kv_cache, 16) || !is_aligned(slot_mapping, 4))
    return MLA_ERR_INVALID_ARGUMENT;
  AppendParams ap;
  ap.rows = static_cast<const uint16_t*>(rows);
  ap.slots = slot_mapping;
  ap.kv = static_cast<uint8_t*>(kv_cache);
  ap.n_slots = (long long)num_blocks * block_size;
  ap.n_tokens = n_tokens;
  ap.inv_scale = 1.0 / static_cast<double>(kv_scale);
  const long long threads = (long long)n_tokens * CHUNKS;
  const dim3 grid(static_cast<unsigned>((threads + APPEND_THREADS - 1) / APPEND_THREADS));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (kv_dtype == MLA_DTYPE_BF16)
    hipLaunchKernelGGL(mla_kv_append_kernel<MLA_DTYPE_BF16>, grid, dim3(APPEND_THREADS), 0, st, ap);
  else
    hipLaunchKernelGGL(mla_kv_append_kernel<MLA_DTYPE_FP8_E4M3FN>, grid, dim3(APPEND_THREADS), 0, st, ap);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
