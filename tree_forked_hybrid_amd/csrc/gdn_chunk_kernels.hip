// Chunked Gated DeltaNet on MFMA (bf16 inputs, dk = dv = 128, chunks of 64 rows).
//
// Per chunk of n <= 64 rows with start state S0 [dv, dk] and g_t = sum_{s<=t} log alpha_s
// (relative to the chunk), the per-token recurrence of "Flide: Accelerating
// Decision Inference with Exact State Forking" §前置知识 is evaluated in closed form:
//     u_t = eta_t (v_t - alpha_t S_{t-1} k_t)                 (so S_t = alpha_t S_{t-1} + u_t k_t^T)
//     (I + A) U = diag(eta) V - diag(eta e^g) K S0^T,          A_ts = eta_t e^{g_t - g_s} k_t.k_s  (s < t)
//     O = diag(e^g) Q S0^T + (Gamma (.) Q K^T) U,              Gamma_ts = e^{g_t - g_s} (s <= t)
//     S_n = e^{g_n} S0 + U^T diag(e^{g_n - g}) K.
// This is the same chunk algebra (Gram matrix, blocked triangular solve by
// forward substitution) as the rollback-free GDN verification of
// "기술 요약: 마진으로부터의 트리 (DFlash-TfM)" 방법론 §3, applied here to plain
// chunks of a segment.  Chunks start at multiples of 64 rows from the segment
// start, so a segment's arithmetic never depends on the rest of the round.
//
// Workgroup = (segment, head), 8 waves.  Wave w owns value channels
// [16w, 16w + 16) and the matching 16 rows of S, which stay in registers for
// the whole segment in the layout the next chunk's MFMA needs as its B operand.
// Everything that depends on those channels (K S0^T, Q S0^T, the solve, O and
// the state update) is wave-local; only the channel-independent pieces (the
// normalised q/k tiles, A, Gamma (.) QK^T and the 16x16 diagonal inverses of
// I + A) are shared through LDS.  MFMA operands are fp16 (q, k are unit
// vectors; the other operands are O(1)), accumulation and the state are fp32.
#include "device_common.hpp"

namespace flide {

int launch_gdn_plain(const MetaView& mv, const flide_gdn_params& p, int phase, const void* x, const float* conv_w,
                     const float* alpha, const float* eta, float* state_pool, void* conv_pool, int32_t n_slots,
                     void* o, void* stream);

namespace {

typedef _Float16 h4v __attribute__((ext_vector_type(4)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int CK = 64;        // chunk rows
constexpr int DK = 128;       // key size
constexpr int DV = 128;       // value size (8 waves x 16 channels)
constexpr int NT = 512;       // threads
constexpr int QS = DK + 8;    // row stride (halves) of the q/k tiles [t][dk]
constexpr int TS = CK + 4;    // row stride (halves) of k^T [dk][t] and of A, P [t][s]
constexpr int DS = 16 + 4;    // row stride (halves) of the diagonal inverses

__device__ __forceinline__ f4v mma16(h4v a, h4v b, f4v c) { return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0); }
__device__ __forceinline__ f4v mma32(h8v a, h8v b, f4v c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

__device__ __forceinline__ h4v to_h4(f4v v) { return h4v{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]}; }
__device__ __forceinline__ h8v cat8(h4v a, h4v b) { return h8v{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }
__device__ __forceinline__ h4v lds4(const _Float16* p) { return *reinterpret_cast<const h4v*>(p); }
__device__ __forceinline__ h8v lds8(const _Float16* p) { return *reinterpret_cast<const h8v*>(p); }

struct ChunkLds {
  _Float16 q[CK * QS];   // normalised q, fp16 (hi part)
  _Float16 k[CK * QS];   // normalised k, fp16 (hi part)
  _Float16 ql[CK * QS];  // q - hi, fp16 (lo part)
  _Float16 kl[CK * QS];  // k - hi, fp16 (lo part)
  float v[CK * DV];      // conv'd values [t][channel]
  _Float16 kt[DK * TS];
  _Float16 a[CK * TS];   // -A (strictly lower blocks)
  _Float16 p[CK * TS];   // Gamma (.) QK^T (lower blocks, diagonal included)
  _Float16 tinv[4 * 16 * DS];
  float a32[4][16][17];  // diagonal blocks of A in fp32 for the inverse
  float g[CK];
  float eta[CK];
  float cw[3 * 128][4];   // conv taps of the head's q, k and v channels (right-aligned: tap 3 = current row)
  float glast;
};

}  // namespace

__global__ void __launch_bounds__(NT) gdn_chunk_kernel(MetaView mv, int phase, int H, int K, int act,
                                                       const bf16_t* __restrict__ x, const float* __restrict__ conv_w,
                                                       const float* __restrict__ alpha,
                                                       const float* __restrict__ eta, float* __restrict__ state_pool,
                                                       bf16_t* __restrict__ conv_pool, int n_slots,
                                                       bf16_t* __restrict__ o) {
  __shared__ ChunkLds L;
  const int item = blockIdx.x, h = blockIdx.y;
  const int R = mv.hdr[H_R];
  int seg;
  if (phase == 0) {
    if (item >= R) return;
    seg = item;
  } else {
    if (item >= mv.hdr[H_NQST]) return;
    seg = R + item;
  }
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g4 = l >> 4;
  const int64_t C = int64_t(H) * (2 * DK + DV);
  const int j = mv.seg_req[seg];
  const int row0 = mv.seg_row0[seg], len = mv.seg_len[seg];
  const int in_slot = mv.seg_state[seg];
  const int out_slot = phase == 0 ? mv.req_out[j] : -1;
  if (in_slot >= n_slots || out_slot >= n_slots || (phase == 1 && in_slot < 0)) {
    if (tid == 0) flag_error(mv.dev_error, E_SLOT);
    return;
  }
  const bf16_t* hist = in_slot >= 0 ? conv_pool + int64_t(in_slot) * (K - 1) * C : nullptr;
  const int qch = h * DK, kch = H * DK + h * DK, vch = 2 * H * DK + h * DV;
  const int ncol = 16 * w + r16;  // this lane's value channel / state row

  // raw inputs of channels (ch, ch+1) at segment-local row u as one dword of two bf16
  // (u < 0: conv history; u >= len or before the history: zero).  Branch-free so that
  // a lane's row loads issue back to back.
  auto pair = [&](int u, int ch) -> uint32_t {
    const bool in_x = u >= 0 && u < len;
    const bool in_h = u < 0 && u >= -(K - 1) && hist != nullptr;
    const bf16_t* ptr = in_x ? x + int64_t(row0 + u) * C + ch
                             : (in_h ? hist + int64_t(K - 1 + u) * C + ch : x + int64_t(row0) * C + ch);
    const uint32_t val = *reinterpret_cast<const uint32_t*>(ptr);
    return (in_x || in_h) ? val : 0u;
  };
  auto lo_f = [](uint32_t v2) { return __uint_as_float(v2 << 16); };
  auto hi_f = [](uint32_t v2) { return __uint_as_float(v2 & 0xFFFF0000u); };

  // state rows [16w, 16w+16) x dk, lane holds S[ncol][16 mb + 4 g4 + i]
  f4v S[8];
  if (in_slot >= 0) {
    const float* src = state_pool + ((int64_t(in_slot) * H + h) * DV + ncol) * DK;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) S[mb] = *reinterpret_cast<const f4v*>(src + 16 * mb + 4 * g4);
  } else {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) S[mb] = f4v{0.f, 0.f, 0.f, 0.f};
  }
  // conv lanes: pass 1 waves 0-3 -> q, 4-7 -> k; pass 2 waves 0-3 -> v; lane = channel pair,
  // wave % 4 = row quarter of the chunk
  const bool is_k = w >= 4;
  const int pair_ch = (is_k ? kch : qch) + 2 * l;
  const int vpair_ch = vch + 2 * l;
  const int quarter = w & 3;
  for (int it = tid; it < 3 * 128 * 4; it += NT) {
    const int ci = it >> 2, tap = it & 3;
    const int ch = ci < DK ? qch + ci : (ci < 2 * DK ? kch + ci - DK : vch + ci - 2 * DK);
    const int tau = tap - (4 - K);
    L.cw[ci][tap] = tau >= 0 ? conv_w[int64_t(ch) * K + tau] : 0.f;
  }
  const int cwq = (is_k ? DK : 0) + 2 * l;  // row of this lane's first q/k channel in L.cw
  const int cwv = 2 * DK + 2 * l;           // row of this lane's first v channel in L.cw

  for (int c0 = 0; c0 < len; c0 += CK) {
    const int n = min(CK, len - c0);
    __syncthreads();  // previous chunk's readers are done with the LDS tiles
    // ---- conv + L2 norm of q and k -> fp16 hi/lo tiles (pass 1) ----
    const int t0 = 16 * quarter;
    for (int half = 0; half < 2; ++half) {
      const int tb = t0 + 8 * half;
      uint32_t rr[11];
#pragma unroll
      for (int i = 0; i < 11; ++i) rr[i] = pair(c0 + tb - 3 + i, pair_ch);
      const float4 wa = *reinterpret_cast<const float4*>(L.cw[cwq]);
      const float4 wb = *reinterpret_cast<const float4*>(L.cw[cwq + 1]);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int t = tb + tt;
        float ya = wa.x * lo_f(rr[tt]) + wa.y * lo_f(rr[tt + 1]) + wa.z * lo_f(rr[tt + 2]) + wa.w * lo_f(rr[tt + 3]);
        float yb = wb.x * hi_f(rr[tt]) + wb.y * hi_f(rr[tt + 1]) + wb.z * hi_f(rr[tt + 2]) + wb.w * hi_f(rr[tt + 3]);
        if (act == 1) {
          ya = ya / (1.f + __expf(-ya));
          yb = yb / (1.f + __expf(-yb));
        }
        const float ss = wave_sum(ya * ya + yb * yb);
        const float inv = t < n ? rsqrtf(ss + 1e-6f) : 0.f;
        const float na = ya * inv, nb = yb * inv;
        const _Float16 ha = (_Float16)na, hb = (_Float16)nb;
        const _Float16 la = (_Float16)(na - (float)ha), lb = (_Float16)(nb - (float)hb);
        _Float16* dst = (is_k ? L.k : L.q) + t * QS + 2 * l;
        _Float16* dsl = (is_k ? L.kl : L.ql) + t * QS + 2 * l;
        dst[0] = ha;
        dst[1] = hb;
        dsl[0] = la;
        dsl[1] = lb;
        if (is_k) {
          L.kt[(2 * l) * TS + t] = ha;
          L.kt[(2 * l + 1) * TS + t] = hb;
        }
      }
    }
    // ---- pass 2: values (waves 0-3); decay and step sizes (wave 4) ----
    if (w < 4) {
     for (int half = 0; half < 2; ++half) {
      const int tb = t0 + 8 * half;
      uint32_t rr[11];
#pragma unroll
      for (int i = 0; i < 11; ++i) rr[i] = pair(c0 + tb - 3 + i, vpair_ch);
      const float4 wa = *reinterpret_cast<const float4*>(L.cw[cwv]);
      const float4 wb = *reinterpret_cast<const float4*>(L.cw[cwv + 1]);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int t = tb + tt;
        float ya = wa.x * lo_f(rr[tt]) + wa.y * lo_f(rr[tt + 1]) + wa.z * lo_f(rr[tt + 2]) + wa.w * lo_f(rr[tt + 3]);
        float yb = wb.x * hi_f(rr[tt]) + wb.y * hi_f(rr[tt + 1]) + wb.z * hi_f(rr[tt + 2]) + wb.w * hi_f(rr[tt + 3]);
        if (act == 1) {
          ya = ya / (1.f + __expf(-ya));
          yb = yb / (1.f + __expf(-yb));
        }
        L.v[t * DV + 2 * l] = t < n ? ya : 0.f;
        L.v[t * DV + 2 * l + 1] = t < n ? yb : 0.f;
      }
     }
    } else if (w == 4) {
      // g = inclusive prefix sum of log alpha over the chunk
      const int t = l;
      const float a = t < n ? alpha[int64_t(row0 + c0 + t) * H + h] : 1.f;
      const float e = t < n ? eta[int64_t(row0 + c0 + t) * H + h] : 0.f;
      float gsum = __logf(a);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float up = __shfl_up(gsum, off, 64);
        if (t >= off) gsum += up;
      }
      L.g[t] = gsum;
      L.eta[t] = e;
      if (t == n - 1) L.glast = gsum;
    }
    __syncthreads();
    // ---- shared products: A = eta_t e^{g_t-g_s} k_t.k_s (s < t), P = e^{g_t-g_s} q_t.k_s (s <= t) ----
    for (int task = w; task < 20; task += 8) {
      const bool isq = task >= 10;
      int blk = isq ? task - 10 : task;  // lower-triangular block index -> (ti, si)
      int ti = 0;
      while (blk > ti) {
        blk -= ti + 1;
        ++ti;
      }
      const int si = blk;
      const int oa = (16 * ti + r16) * QS + 8 * g4, ob = (16 * si + r16) * QS + 8 * g4;
      f4v acc = {0.f, 0.f, 0.f, 0.f};
      if (isq) {
        // q.k of unit vectors can be far smaller than its rounding error in fp16: hi*hi + hi*lo + lo*hi
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const h8v qh = lds8(L.q + oa + 32 * c), kh = lds8(L.k + ob + 32 * c);
          acc = mma32(qh, kh, acc);
          acc = mma32(qh, lds8(L.kl + ob + 32 * c), acc);
          acc = mma32(lds8(L.ql + oa + 32 * c), kh, acc);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc = mma32(lds8(L.k + oa + 32 * c), lds8(L.k + ob + 32 * c), acc);
      }
      const int s = 16 * si + r16;
      const float gs = L.g[s];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * ti + 4 * g4 + i;
        const float dec = __expf(L.g[t] - gs);
        if (isq) {
          L.p[t * TS + s] = (_Float16)(s <= t ? dec * acc[i] : 0.f);
        } else {
          const float av = s < t ? L.eta[t] * dec * acc[i] : 0.f;
          L.a[t * TS + s] = (_Float16)(-av);
          if (ti == si) L.a32[ti][4 * g4 + i][r16] = av;
        }
      }
    }
    __syncthreads();
    // ---- diagonal inverses T_bb = (I + A_bb)^{-1} by forward substitution (waves 0-3) ----
    if (w < 4) {
      const int b = w, col = r16, part = g4;
      float tv[4] = {0.f, 0.f, 0.f, 0.f};  // T[part + 4k][col]
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int jj = part + 4 * kk;
          if (jj < r) acc += L.a32[b][r][jj] * tv[kk];
        }
        acc += __shfl_xor(acc, 16, 64);
        acc += __shfl_xor(acc, 32, 64);
        const float trc = (r == col ? 1.f : 0.f) - acc;
        if ((r & 3) == part) tv[r >> 2] = trc;
        if (part == 0) L.tinv[(b * 16 + r) * DS + col] = (_Float16)trc;
      }
    }
    // ---- wave-local, channel-dependent work part 1 (no dependency on the inverses) ----
    h8v sf[4];  // S as the B operand of K S^T / Q S^T (k-slots permuted to match the register layout)
#pragma unroll
    for (int c = 0; c < 4; ++c) sf[c] = cat8(to_h4(S[2 * c]), to_h4(S[2 * c + 1]));
    f4v ks[4], qs[4], rhs[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      ks[rb] = f4v{0.f, 0.f, 0.f, 0.f};
      qs[rb] = f4v{0.f, 0.f, 0.f, 0.f};
      const _Float16* kr = L.k + (16 * rb + r16) * QS + 4 * g4;
      const _Float16* qr = L.q + (16 * rb + r16) * QS + 4 * g4;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        ks[rb] = mma32(cat8(lds4(kr + 32 * c), lds4(kr + 32 * c + 16)), sf[c], ks[rb]);
        qs[rb] = mma32(cat8(lds4(qr + 32 * c), lds4(qr + 32 * c + 16)), sf[c], qs[rb]);
      }
      // values of this lane's channel (conv) and the right-hand side
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * rb + 4 * g4 + i;
        const float vv = L.v[t * DV + ncol];
        const float e = L.eta[t];
        rhs[rb][i] = e * (vv - __expf(L.g[t]) * ks[rb][i]);
      }
    }
    __syncthreads();  // diagonal inverses ready
    // ---- blocked forward substitution U = (I + A)^{-1} RHS ----
    h4v uh[4];
    f4v u[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f4v acc = rhs[rb];
#pragma unroll
      for (int jb = 0; jb < rb; ++jb) acc = mma16(lds4(L.a + (16 * rb + r16) * TS + 16 * jb + 4 * g4), uh[jb], acc);
      u[rb] = mma16(lds4(L.tinv + (rb * 16 + r16) * DS + 4 * g4), to_h4(acc), f4v{0.f, 0.f, 0.f, 0.f});
      uh[rb] = to_h4(u[rb]);
    }
    // ---- outputs O = e^g Q S0^T + P U ----
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f4v acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __expf(L.g[16 * rb + 4 * g4 + i]) * qs[rb][i];
#pragma unroll
      for (int jb = 0; jb <= rb; ++jb) acc = mma16(lds4(L.p + (16 * rb + r16) * TS + 16 * jb + 4 * g4), uh[jb], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * rb + 4 * g4 + i;
        if (t < n) o[(int64_t(row0 + c0 + t) * H + h) * DV + ncol] = f32_to_bf16(acc[i]);
      }
    }
    // ---- state update S = e^{g_n} S + U^T diag(e^{g_n - g}) K ----
    const float gl = L.glast;
    h4v ud[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f4v v4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * rb + 4 * g4 + i;
        v4[i] = t < n ? __expf(gl - L.g[t]) * u[rb][i] : 0.f;
      }
      ud[rb] = to_h4(v4);
    }
    const float egl = __expf(gl);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      f4v acc = S[mb] * egl;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc = mma16(lds4(L.kt + (16 * mb + r16) * TS + 16 * rb + 4 * g4), ud[rb], acc);
      S[mb] = acc;
    }
  }

  if (phase == 0) {
    float* dst = state_pool + ((int64_t(out_slot) * H + h) * DV + ncol) * DK;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) *reinterpret_cast<f4v*>(dst + 16 * mb + 4 * g4) = S[mb];
    // conv window: last K-1 raw inputs of (history ++ segment) over the head's q, k and v channels
    bf16_t* wdst = conv_pool + int64_t(out_slot) * (K - 1) * C;
    const int nch = 2 * DK + DV;
    for (int it = tid; it < (K - 1) * nch; it += NT) {
      const int wr = it / nch, ci = it - wr * nch;
      const int ch = ci < DK ? qch + ci : (ci < 2 * DK ? kch + ci - DK : vch + ci - 2 * DK);
      const int u = len - (K - 1) + wr;
      bf16_t val = 0;
      if (u >= 0)
        val = x[int64_t(row0 + u) * C + ch];
      else if (hist != nullptr)
        val = hist[int64_t(K - 1 + u) * C + ch];
      wdst[int64_t(wr) * C + ch] = val;
    }
  }
}

bool gdn_uses_chunk(const flide_gdn_params& p) { return p.dtype == FLIDE_BF16 && p.dk == DK && p.dv == DV; }

int launch_gdn(const MetaView& mv, const flide_gdn_params& p, int phase, const void* x, const float* conv_w,
               const float* alpha, const float* eta, float* state_pool, void* conv_pool, int32_t n_slots, void* o,
               void* stream) {
  if (!gdn_uses_chunk(p))
    return launch_gdn_plain(mv, p, phase, x, conv_w, alpha, eta, state_pool, conv_pool, n_slots, o, stream);
  dim3 grid(phase == 0 ? mv.R_cap : (mv.Q_cap > 0 ? mv.Q_cap : 1), p.H);
  hipLaunchKernelGGL(gdn_chunk_kernel, grid, dim3(NT), 0, (hipStream_t)stream, mv, phase, p.H, p.conv_k, p.act,
                     (const bf16_t*)x, conv_w, alpha, eta, state_pool, (bf16_t*)conv_pool, n_slots, (bf16_t*)o);
  return int(hipGetLastError());
}

}  // namespace flide
