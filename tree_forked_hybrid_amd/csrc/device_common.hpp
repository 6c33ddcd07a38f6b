// Device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flide_internal.hpp"

namespace flide {

typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round to nearest even (inputs here are finite).
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Two floats to two bf16 (round to nearest even, v_cvt_pk_bf16_f32); lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2v));
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return bf16_t(u >> 16);
}

template <typename T>
__device__ __forceinline__ float load_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_f32<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ void store_f32(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_f32<float>(float* p, int64_t i, float v) {
  p[i] = v;
}
template <>
__device__ __forceinline__ void store_f32<bf16_t>(bf16_t* p, int64_t i, float v) {
  p[i] = f32_to_bf16(v);
}

// Sum / max over the four 16-lane rows of a wave (lane l with lanes l ^ 16, l ^ 32, l ^ 48) on the
// VALU: v_permlane16_swap / v_permlane32_swap pair each lane with the same lane of the partner row,
// and combining both halves of a swap gives the pair result.  Same pairing as a shuffle butterfly
// (xor 16, then xor 32), so the results match it bit for bit.
__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// One direct-to-LDS buffer load per lane of BYTES (4 or 16): lane i writes bytes [BYTES i, BYTES i + BYTES)
// after the wave-uniform LDS byte address lds_addr, read at byte offset voff of the resource (zeros where
// voff is outside it).  Written as inline asm so that the compiler does not track the copy: it would
// otherwise make every later LDS access it cannot tell apart from the destination wait for it, while
// the kernels wait for their copies explicitly (vmcnt), one stage later.  M0 is written here and used
// by nothing else; the nops cover the SGPR-write and M0-write hazards.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 in the clobber list is intended
template <int BYTES>
__device__ __forceinline__ void dma_to_lds(__amdgpu_buffer_rsrc_t r, unsigned lds_addr, int voff) {
  static_assert(BYTES == 4 || BYTES == 16, "dword or dwordx4 copies");
  if (BYTES == 16)
    asm volatile("s_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 :: "v"(voff), "s"(lds_addr), "s"(r) : "memory", "m0");
  else
    asm volatile("s_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 1\n\tbuffer_load_dword %0, %2, 0 offen lds"
                 :: "v"(voff), "s"(lds_addr), "s"(r) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void flag_error(int32_t* dev_error, int32_t bit) { atomicOr(dev_error, bit); }

// Stream row -> segment index: the last segment whose first row is <= row.
// Segments are ordered by first row; empty segments never shadow the row's segment.
__device__ __forceinline__ int find_segment(const int32_t* seg_row0, int n_seg, int row) {
  int lo = 0, hi = n_seg - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (seg_row0[mid] <= row)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

}  // namespace flide
