// Matrix-core rate at the running clock, for roofline reporting: the
// datasheet peak assumes the nominal clock, while a long MFMA-dense launch on
// this part runs power-limited below it.  Every wave issues the instruction
// the attention kernels use for the element type, over four independent
// accumulators (so no product waits for the previous one), in a loop of a
// fixed length; a workgroup holds two such waves per SIMD and reserves 96 KB
// of the CU's 160 KB of LDS, so no second workgroup fits beside it and a
// launch of one workgroup per CU spreads evenly over the CUs.  Nothing
// else runs in the loop: the figure is the rate the matrix cores reach on
// their own, the ceiling the attention kernels are measured against.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vlp.h"

namespace vlp {
namespace {

typedef __bf16 cal_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 cal_f16x8 __attribute__((ext_vector_type(8)));
typedef float cal_f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t cal_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCalThreads = 512;  // eight waves: two per SIMD
constexpr int kCalChains = 4;     // independent accumulators per wave
constexpr int kCalReserveFloats = 96 * 1024 / 4;

// Flops of one instruction: 2 * M * N * K.
constexpr double kFlops16 = 2.0 * 32 * 32 * 16;  // 32x32x16 bf16 / fp16
constexpr double kFlops32 = 2.0 * 32 * 32 * 2;   // 32x32x2 fp32

template <int DT>
__global__ __launch_bounds__(kCalThreads) void mfma_rate_kernel(int iters, float* __restrict__ sink) {
  __shared__ float reserve[kCalReserveFloats];
  const uint32_t t = threadIdx.x;
  cal_f32x16 acc[kCalChains];
#pragma unroll
  for (int c = 0; c < kCalChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  if constexpr (DT == VLP_FP32) {
    const float a = 1.0f + 1e-3f * static_cast<float>(t & 7);
    const float b = 1.0f - 1e-3f * static_cast<float>(t >> 6);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < kCalChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[c], 0, 0, 0);
    }
  } else {
    // small normal values of either 16-bit format, varied per lane
    cal_u32x4 a, b;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[j] = 0x3c003c00u + ((t + j) & 7);
      b[j] = 0x3c003c00u + ((t >> 3) & 7) + j;
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < kCalChains; ++c) {
        if constexpr (DT == VLP_BF16)
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(cal_bf16x8, a),
                                                           __builtin_bit_cast(cal_bf16x8, b), acc[c], 0, 0, 0);
        else
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(cal_f16x8, a),
                                                          __builtin_bit_cast(cal_f16x8, b), acc[c], 0, 0, 0);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kCalChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (iters < 0) {  // never taken (iters >= 1); the use keeps the LDS reservation
    reserve[t] = s;
    __syncthreads();
    s = reserve[kCalReserveFloats - 1 - t];
  }
  sink[static_cast<size_t>(blockIdx.x) * kCalThreads + t] = s;  // keeps the products live
}

}  // namespace

// Flops of one launch of launch_mfma_rate.
double mfma_rate_flops(int dtype, int blocks, int iters) {
  return (dtype == VLP_FP32 ? kFlops32 : kFlops16) * kCalChains * (kCalThreads / 64) * static_cast<double>(blocks) *
         iters;
}

hipError_t launch_mfma_rate(int dtype, int blocks, int iters, float* sink, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(blocks)), block(kCalThreads);
  if (dtype == VLP_FP32)
    hipLaunchKernelGGL(mfma_rate_kernel<VLP_FP32>, grid, block, 0, s, iters, sink);
  else if (dtype == VLP_FP16)
    hipLaunchKernelGGL(mfma_rate_kernel<VLP_FP16>, grid, block, 0, s, iters, sink);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<VLP_BF16>, grid, block, 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace vlp
