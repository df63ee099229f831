// Achievable-peak probe: the matrix-core shapes of the decode kernels with
// every CU busy (a measurement hook, declared in include/mla_probe.h).
#include <hip/hip_runtime.h>

#include "mla_probe.h"

namespace {

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float f32x4_p __attribute__((ext_vector_type(4)));
typedef float f32x16_p __attribute__((ext_vector_type(16)));
typedef int i32x8_p __attribute__((ext_vector_type(8)));

constexpr int THREADS = MLA_PROBE_THREADS;
constexpr int CHAINS = MLA_PROBE_CHAINS;

// M, N, K and accumulator elements per lane of each shape
struct ShapeInfo {
  int m, n, k, per_lane;
};
constexpr ShapeInfo SHAPES[3] = {{16, 16, 32, 4}, {32, 32, 16, 16}, {16, 16, 128, 4}};

template <int SHAPE>
__global__ __launch_bounds__(THREADS) void mla_probe_mfma_kernel(int iters, float x, float* out) {
  float sum = 0.f;
  if constexpr (SHAPE == MLA_PROBE_MFMA_16X16X128_FP8) {
    // four e4m3fn codes of x per dword (exact for powers of two in range)
    const int c4 = __builtin_amdgcn_cvt_pk_fp8_f32(x, x, __builtin_amdgcn_cvt_pk_fp8_f32(x, x, 0, false), true);
    i32x8_p a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = c4;
    f32x4_p acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = f32x4_p{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < CHAINS; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, a, acc[c], 0, 0, 0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) sum += acc[c][e];
  } else {
    const __bf16 xb = static_cast<__bf16>(x);
    bf16x8_p a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = xb;
    if constexpr (SHAPE == MLA_PROBE_MFMA_16X16X32_BF16) {
      f32x4_p acc[CHAINS];
#pragma unroll
      for (int c = 0; c < CHAINS; ++c) acc[c] = f32x4_p{0.f, 0.f, 0.f, 0.f};
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, acc[c], 0, 0, 0);
      }
#pragma unroll
      for (int c = 0; c < CHAINS; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) sum += acc[c][e];
    } else {
      f32x16_p acc[CHAINS];
#pragma unroll
      for (int c = 0; c < CHAINS; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[c], 0, 0, 0);
      }
#pragma unroll
      for (int c = 0; c < CHAINS; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += acc[c][e];
    }
  }
  out[(size_t)blockIdx.x * THREADS + threadIdx.x] = sum;
}

bool shape_ok(int32_t shape) { return shape >= 0 && shape <= 2; }

}  // namespace

extern "C" double mla_probe_mfma_flops(int32_t shape, int32_t workgroups, int32_t iters) {
  if (!shape_ok(shape) || workgroups < 1 || iters < 1) return 0.0;
  const ShapeInfo& s = SHAPES[shape];
  return (double)workgroups * (THREADS / 64) * iters * CHAINS * 2.0 * s.m * s.n * s.k;
}

extern "C" double mla_probe_mfma_expected(int32_t shape, int32_t iters, float x) {
  if (!shape_ok(shape)) return 0.0;
  const ShapeInfo& s = SHAPES[shape];
  return (double)CHAINS * s.per_lane * iters * s.k * (double)x * (double)x;
}

extern "C" int32_t mla_probe_mfma(int32_t shape, int32_t workgroups, int32_t iters, float x,
                                  float* out, void* stream) {
  if (!shape_ok(shape) || workgroups < 1 || workgroups > (1 << 20) || iters < 1 ||
      iters > (1 << 24) || out == nullptr)
    return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(workgroups)), block(THREADS);
  if (shape == MLA_PROBE_MFMA_16X16X32_BF16)
    hipLaunchKernelGGL(mla_probe_mfma_kernel<MLA_PROBE_MFMA_16X16X32_BF16>, grid, block, 0, st, iters, x, out);
  else if (shape == MLA_PROBE_MFMA_32X32X16_BF16)
    hipLaunchKernelGGL(mla_probe_mfma_kernel<MLA_PROBE_MFMA_32X32X16_BF16>, grid, block, 0, st, iters, x, out);
  else
    hipLaunchKernelGGL(mla_probe_mfma_kernel<MLA_PROBE_MFMA_16X16X128_FP8>, grid, block, 0, st, iters, x, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
