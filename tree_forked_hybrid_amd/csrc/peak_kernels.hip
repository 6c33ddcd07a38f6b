// Measured ceiling of the bf16 matrix cores, reported beside the published peak: a loop of independent
// v_mfma_f32_16x16x32_bf16 products, eight accumulators per wave, 512 workgroups of four waves (on
// average two waves per SIMD, the occupancy of the attention kernel).  The products are written as asm
// so that the eight accumulators stay in place (the compiler's allocation of this loop shuffles them);
// successive products of one accumulator are eight instructions apart, and the accumulators are read
// only after a wait longer than the longest product.
#include <hip/hip_runtime.h>

#include "flide_internal.hpp"

namespace flide {

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

__device__ float g_peak_sink;  // written only when the sum is exactly -1, which keeps the loop alive

constexpr int kPeakBlocks = 512;
constexpr int kPeakThreads = 256;

__global__ void __launch_bounds__(kPeakThreads) mfma_peak_kernel(int iters) {
  const int l = threadIdx.x & 63;
  b8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * float(l + i));
    b[i] = (__bf16)(0.002f * float(l - i));
  }
  f4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  asm volatile("s_nop 4" : "+v"(a), "+v"(b));  // the operands' last vector writes are done
  for (int it = 0; it < iters; ++it) {
    asm volatile(
        "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
        "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
        "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
        "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7"
        : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
        : "v"(a), "v"(b));
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5),
               "+v"(c6), "+v"(c7));
  const float r = c0[0] + c1[1] + c2[2] + c3[3] + c4[0] + c5[1] + c6[2] + c7[3];
  if (r == -1.f) g_peak_sink = r;
}

}  // namespace

}  // namespace flide

extern "C" flide_status flide_measure_mfma_peak(int32_t iters, void* stream, double* tflops) {
  if (iters < 1 || tflops == nullptr) return FLIDE_E_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess) return FLIDE_E_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return FLIDE_E_HIP;
  }
  flide_status status = FLIDE_OK;
  // one short launch first: clocks and code object warm
  hipLaunchKernelGGL(flide::mfma_peak_kernel, dim3(flide::kPeakBlocks), dim3(flide::kPeakThreads), 0, st, 64);
  if (hipEventRecord(e0, st) != hipSuccess) status = FLIDE_E_HIP;
  hipLaunchKernelGGL(flide::mfma_peak_kernel, dim3(flide::kPeakBlocks), dim3(flide::kPeakThreads), 0, st, iters);
  if (status == FLIDE_OK && (hipGetLastError() != hipSuccess || hipEventRecord(e1, st) != hipSuccess ||
                             hipEventSynchronize(e1) != hipSuccess))
    status = FLIDE_E_HIP;
  float ms = 0.f;
  if (status == FLIDE_OK && (hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0.f)) status = FLIDE_E_HIP;
  if (status == FLIDE_OK) {
    const double flop = double(flide::kPeakBlocks) * (flide::kPeakThreads / 64) * double(iters) * 8.0 * 16 * 16 * 32 * 2;
    *tflops = flop / (double(ms) * 1e-3) / 1e12;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return status;
}
