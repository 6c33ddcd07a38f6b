// Selective readout, Eq. (1): p_i(o) = exp(w_o^T h_i) / sum_{o' in O_i} exp(w_o'^T h_i)
// on question-final rows only (Korean summary §어떻게 동작하나; "Flide:
// Accelerating Decision Inference with Exact State Forking" §方法步骤详情,
// fourth step).
//
// One wave per question: the hidden row is read once into registers, each
// option row is streamed with 16-byte loads and reduced across the wave in
// fp32; the softmax over the (few) options is done by the same wave.
#include "device_common.hpp"

namespace flide {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* out);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* out) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* out) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// hidden must be a multiple of 8 and at most 64 * 8 * kMaxChunks.
constexpr int kMaxChunks = 16;  // hidden <= 8192

template <typename T>
__global__ void __launch_bounds__(256) readout_kernel(MetaView mv, int hidden, const T* __restrict__ h,
                                                      const T* __restrict__ w_opt,
                                                      const int32_t* __restrict__ opt_off,
                                                      const int32_t* __restrict__ opt_id, int n_opt_rows,
                                                      float* __restrict__ probs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int qi = blockIdx.x * 4 + wave;
  if (qi >= mv.hdr[H_NQST]) return;
  const int row = mv.qfin_row[qi];
  if (row < 0 || row >= mv.hdr[H_T]) {
    if (lane == 0) flag_error(mv.dev_error, E_SEGMENT);
    return;
  }
  const int chunks = hidden / 8;  // 8 elements per lane per chunk
  float hv[kMaxChunks][8];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int idx = (c * 64 + lane) * 8;
    if (c * 64 + lane < chunks) {
      load8(h + int64_t(row) * hidden + idx, hv[c]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[c][e] = 0.f;
    }
  }
  const int o0 = opt_off[qi], o1 = opt_off[qi + 1];
  // logits with a running max and a rescaled running sum (every lane holds the
  // wave-reduced values).  Options go in batches of eight: their row loads and
  // wave reductions are independent, so a batch waits for one memory round trip
  // instead of one per option.  A question with at most one batch of options
  // keeps its logits in registers; with more, lane 0 stores the logits and later
  // normalises them itself (no lane reads another lane's global store).
  constexpr int OB = 8;
  const bool one_batch = o1 - o0 <= OB;
  float lg[OB];
  float zmax = -INFINITY, se = 0.f;
  for (int kb = o0; kb < o1; kb += OB) {
    int orow[OB];
    bool ok[OB];
#pragma unroll
    for (int j = 0; j < OB; ++j) {
      orow[j] = kb + j < o1 ? opt_id[kb + j] : 0;
      ok[j] = kb + j < o1 && orow[j] >= 0 && orow[j] < n_opt_rows;
    }
    float acc[OB] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      if (c * 64 + lane < chunks) {
#pragma unroll
        for (int j = 0; j < OB; ++j) {
          if (!ok[j]) continue;
          float wv[8];
          load8(w_opt + int64_t(orow[j]) * hidden + (c * 64 + lane) * 8, wv);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[j] += hv[c][e] * wv[e];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < OB; ++j) acc[j] = wave_sum(acc[j]);
#pragma unroll
    for (int j = 0; j < OB; ++j) {
      const int k = kb + j;
      if (k >= o1) break;
      lg[j] = ok[j] ? acc[j] : -INFINITY;
      if (!ok[j]) {
        if (lane == 0) {
          flag_error(mv.dev_error, E_OPTION);
          if (!one_batch) probs[k] = -INFINITY;
        }
        continue;
      }
      const float znew = fmaxf(zmax, acc[j]);
      se = (zmax == -INFINITY ? 0.f : se * __expf(zmax - znew)) + __expf(acc[j] - znew);
      zmax = znew;
      if (lane == 0 && !one_batch) probs[k] = acc[j];
    }
  }
  if (lane == 0) {
    const float inv = se > 0.f ? 1.f / se : 0.f;
    if (one_batch) {
#pragma unroll
      for (int j = 0; j < OB; ++j)
        if (o0 + j < o1) probs[o0 + j] = __expf(lg[j] - zmax) * inv;
    } else {
      for (int k = o0; k < o1; ++k) probs[k] = __expf(probs[k] - zmax) * inv;
    }
  }
}

int launch_readout(const MetaView& mv, const flide_readout_params& p, const void* h, const void* w_opt,
                   const int32_t* opt_off, const int32_t* opt_id, int32_t n_opt_rows, float* probs,
                   void* stream) {
  const int blocks = mv.Q_cap > 0 ? (mv.Q_cap + 3) / 4 : 1;
  if (p.dtype == FLIDE_BF16)
    hipLaunchKernelGGL(readout_kernel<bf16_t>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, mv, p.hidden,
                       (const bf16_t*)h, (const bf16_t*)w_opt, opt_off, opt_id, n_opt_rows, probs);
  else
    hipLaunchKernelGGL(readout_kernel<float>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, mv, p.hidden,
                       (const float*)h, (const float*)w_opt, opt_off, opt_id, n_opt_rows, probs);
  return int(hipGetLastError());
}

}  // namespace flide
