// Gated DeltaNet layer over the flat stream, in two calls.
//
// Layer ("Flide: Accelerating Decision Inference with Exact State Forking"
// §前置知识): a short causal conv, then per head
//     S_t = alpha_t S_{t-1} (I - eta_t k_t k_t^T) + eta_t v_t k_t^T,   o_t = S_t q_t.
// Two calls (same page §方法步骤详情; Korean summary §무엇과 다른가): call 0 runs
// every trunk and leaves S_P and the conv window of each request in its output
// slot; call 1 runs every question segment at once, each starting from the slot
// its segment's state index names — a read by index, never a copy — with the
// first conv taps of every question reading that slot's trunk tail.
//
// Work item = (segment, head, block of d_v rows of S).  Rows of S are
// independent under the recurrence (the update multiplies S on the right), so
// splitting d_v is exact and keeps every summation order fixed: the result
// bits of a segment never depend on the rest of the round.
#include "device_common.hpp"

namespace flide {

constexpr int kGdnThreads = 256;
constexpr int kGdnStage = 32;  // tokens staged per pass (conv + norms in parallel)

// Raw input of channel `ch` at segment-local index u (u < 0: conv history).
template <typename T>
__device__ __forceinline__ float gdn_raw(const T* __restrict__ x, const T* __restrict__ hist, int64_t C, int K,
                                         int row0, int u, int ch) {
  if (u >= 0) return load_f32(x, int64_t(row0 + u) * C + ch);
  if (hist == nullptr) return 0.f;
  return load_f32(hist, int64_t(K - 1 + u) * C + ch);
}

// Plain per-token kernel: the state block lives in registers (row r of the
// block per group of TPR lanes, TPR columns interleaved per lane); conv and
// L2 norms for kGdnStage tokens are computed in parallel into LDS first.
template <typename T, int DK, int DB>
__global__ void __launch_bounds__(kGdnThreads) gdn_plain_kernel(MetaView mv, int phase, int H, int DV, int K,
                                                                 int act, const T* __restrict__ x,
                                                                 const float* __restrict__ conv_w,
                                                                 const float* __restrict__ alpha,
                                                                 const float* __restrict__ eta,
                                                                 float* __restrict__ state_pool,
                                                                 T* __restrict__ conv_pool, int n_slots,
                                                                 T* __restrict__ o) {
  constexpr int TPR = kGdnThreads / DB;  // lanes per state row
  constexpr int CPT = DK / TPR;          // columns per lane
  static_assert(TPR * DB == kGdnThreads && CPT * TPR == DK && TPR <= 64, "bad GDN tiling");
  __shared__ float yq[kGdnStage][DK];
  __shared__ float yk[kGdnStage][DK];
  __shared__ float yv[kGdnStage][DB];
  __shared__ float s_alpha[kGdnStage], s_eta[kGdnStage], s_rq[kGdnStage], s_rk[kGdnStage];

  const int item = blockIdx.x;
  const int h = blockIdx.y;
  const int blk = blockIdx.z;
  const int R = mv.hdr[H_R];
  int seg;
  if (phase == 0) {
    if (item >= R) return;
    seg = item;
  } else {
    if (item >= mv.hdr[H_NQST]) return;
    seg = R + item;
  }
  const int tid = threadIdx.x;
  const int r = tid / TPR;   // state row within the block
  const int cl = tid % TPR;  // column lane
  const int64_t C = int64_t(H) * (2 * DK + DV);
  const int j = mv.seg_req[seg];
  const int row0 = mv.seg_row0[seg];
  const int len = mv.seg_len[seg];
  int in_slot = mv.seg_state[seg];  // -1: zero state and zero history
  const int out_slot = phase == 0 ? mv.req_out[j] : -1;
  // an interior checkpoint of the trunk: its slot and the segment rows it covers
  const int save_slot = phase == 0 ? mv.req_save_slot[j] : -1;
  const int save_rows = save_slot >= 0 ? mv.req_save_m[j] - mv.req_m[j] : -1;
  if (in_slot >= n_slots || out_slot >= n_slots || save_slot >= n_slots || (phase == 1 && in_slot < 0)) {
    if (tid == 0) flag_error(mv.dev_error, E_SLOT);
    return;
  }
  const T* hist = in_slot >= 0 ? conv_pool + int64_t(in_slot) * (K - 1) * C : nullptr;
  const int qch = h * DK, kch = H * DK + h * DK, vch = 2 * H * DK + h * DV + blk * DB;

  float S[CPT];
  if (in_slot >= 0) {
    const float* src = state_pool + ((int64_t(in_slot) * H + h) * DV + blk * DB + r) * DK;
#pragma unroll
    for (int i = 0; i < CPT; ++i) S[i] = src[cl + TPR * i];
  } else {
#pragma unroll
    for (int i = 0; i < CPT; ++i) S[i] = 0.f;
  }

  for (int c0 = 0; c0 < len; c0 += kGdnStage) {
    const int n = min(kGdnStage, len - c0);
    // conv (+ optional SiLU) for the staged tokens: q, k channels of head h and this block's v channels
    constexpr int NCH = 2 * DK + DB;
    for (int w = tid; w < n * NCH; w += kGdnThreads) {
      const int t = w / NCH, cidx = w - t * NCH;
      int ch;
      float* dst;
      if (cidx < DK) {
        ch = qch + cidx;
        dst = &yq[t][cidx];
      } else if (cidx < 2 * DK) {
        ch = kch + cidx - DK;
        dst = &yk[t][cidx - DK];
      } else {
        ch = vch + cidx - 2 * DK;
        dst = &yv[t][cidx - 2 * DK];
      }
      float acc = 0.f;
      for (int tau = 0; tau < K; ++tau)
        acc += conv_w[int64_t(ch) * K + tau] * gdn_raw(x, hist, C, K, row0, c0 + t - (K - 1) + tau, ch);
      if (act == 1) acc = acc / (1.f + __expf(-acc));
      *dst = acc;
    }
    for (int t = tid; t < n; t += kGdnThreads) {
      s_alpha[t] = alpha[int64_t(row0 + c0 + t) * H + h];
      s_eta[t] = eta[int64_t(row0 + c0 + t) * H + h];
    }
    __syncthreads();
    // inverse L2 norms of q and k: 4 lanes per (token, q|k)
    for (int w = tid; w < n * 8; w += kGdnThreads) {
      const int t = w >> 3, which = (w >> 2) & 1, part = w & 3;
      const float* src = which ? yk[t] : yq[t];
      float ss = 0.f;
      for (int c = part; c < DK; c += 4) ss += src[c] * src[c];
      ss += __shfl_xor(ss, 1, 64);
      ss += __shfl_xor(ss, 2, 64);
      if (part == 0) {
        float inv = rsqrtf(ss + 1e-6f);
        if (which)
          s_rk[t] = inv;
        else
          s_rq[t] = inv;
      }
    }
    __syncthreads();
    // the recurrence, token by token: S <- alpha S + eta (v - alpha S k) k^T, o = S q
    for (int t = 0; t < n; ++t) {
      const float a = s_alpha[t], e = s_eta[t], rk = s_rk[t], rq = s_rq[t];
      float kk[CPT];
      float sk = 0.f;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        kk[i] = yk[t][cl + TPR * i] * rk;
        sk += S[i] * kk[i];
      }
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) sk += __shfl_xor(sk, off, 64);
      const float u = e * (yv[t][r] - a * sk);
      float so = 0.f;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        S[i] = a * S[i] + u * kk[i];
        so += S[i] * (yq[t][cl + TPR * i] * rq);
      }
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) so += __shfl_xor(so, off, 64);
      if (cl == 0) store_f32(o, (int64_t(row0 + c0 + t) * H + h) * DV + blk * DB + r, so);
      if (c0 + t + 1 == save_rows) {  // the checkpoint's state: S after this row
        float* sdst = state_pool + ((int64_t(save_slot) * H + h) * DV + blk * DB + r) * DK;
#pragma unroll
        for (int i = 0; i < CPT; ++i) sdst[cl + TPR * i] = S[i];
      }
    }
    __syncthreads();
  }

  if (phase == 0) {
    float* dst = state_pool + ((int64_t(out_slot) * H + h) * DV + blk * DB + r) * DK;
#pragma unroll
    for (int i = 0; i < CPT; ++i) dst[cl + TPR * i] = S[i];
    // conv window: the K-1 raw inputs of (history ++ segment) before segment row `upto`; q/k channels
    // by block 0 only; for the trunk's end and for an interior checkpoint
    auto write_window = [&](int slot, int upto) {
      T* wdst = conv_pool + int64_t(slot) * (K - 1) * C;
      const int nch = (blk == 0 ? 2 * DK : 0) + DB;
      for (int w = tid; w < (K - 1) * nch; w += kGdnThreads) {
        const int wr = w / nch, ci = w - wr * nch;
        int ch;
        if (blk == 0 && ci < DK)
          ch = qch + ci;
        else if (blk == 0 && ci < 2 * DK)
          ch = kch + ci - DK;
        else
          ch = vch + ci - (blk == 0 ? 2 * DK : 0);
        const float val = gdn_raw(x, hist, C, K, row0, upto - (K - 1) + wr, ch);
        store_f32(wdst, int64_t(wr) * C + ch, val);
      }
    };
    write_window(out_slot, len);
    if (save_slot >= 0) write_window(save_slot, save_rows);
  }
}

template <typename T, int DK, int DB>
static int launch_plain(const MetaView& mv, const flide_gdn_params& p, int phase, const void* x,
                        const float* conv_w, const float* alpha, const float* eta, float* state_pool,
                        void* conv_pool, int32_t n_slots, void* o, void* stream) {
  dim3 grid(phase == 0 ? mv.R_cap : (mv.Q_cap > 0 ? mv.Q_cap : 1), p.H, p.dv / DB);
  hipLaunchKernelGGL((gdn_plain_kernel<T, DK, DB>), grid, dim3(kGdnThreads), 0, (hipStream_t)stream, mv, phase,
                     p.H, p.dv, p.conv_k, p.act, (const T*)x, conv_w, alpha, eta, state_pool, (T*)conv_pool,
                     n_slots, (T*)o);
  return int(hipGetLastError());
}

template <typename T>
static int dispatch_plain(const MetaView& mv, const flide_gdn_params& p, int phase, const void* x,
                          const float* conv_w, const float* alpha, const float* eta, float* state_pool,
                          void* conv_pool, int32_t n_slots, void* o, void* stream) {
  const int db = p.dv >= 32 ? 32 : p.dv;
#define FLIDE_GDN_CASE(DKV, DBV)                                                                             \
  if (p.dk == DKV && db == DBV)                                                                             \
    return launch_plain<T, DKV, DBV>(mv, p, phase, x, conv_w, alpha, eta, state_pool, conv_pool, n_slots, o, \
                                     stream);
  FLIDE_GDN_CASE(128, 32)
  FLIDE_GDN_CASE(64, 32)
  FLIDE_GDN_CASE(32, 32)
  FLIDE_GDN_CASE(128, 16)
  FLIDE_GDN_CASE(64, 16)
  FLIDE_GDN_CASE(32, 16)
  FLIDE_GDN_CASE(16, 16)
#undef FLIDE_GDN_CASE
  return int(hipErrorInvalidValue);
}

int launch_gdn_plain(const MetaView& mv, const flide_gdn_params& p, int phase, const void* x, const float* conv_w,
               const float* alpha, const float* eta, float* state_pool, void* conv_pool, int32_t n_slots, void* o,
               void* stream) {
  if (p.dtype == FLIDE_BF16)
    return dispatch_plain<bf16_t>(mv, p, phase, x, conv_w, alpha, eta, state_pool, conv_pool, n_slots, o, stream);
  return dispatch_plain<float>(mv, p, phase, x, conv_w, alpha, eta, state_pool, conv_pool, n_slots, o, stream);
}

}  // namespace flide
