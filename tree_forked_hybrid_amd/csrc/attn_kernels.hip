// Tree-masked varlen attention over the flat stream.
//
// Visibility ("Flide: Accelerating Decision Inference with Exact State
// Forking" §方法步骤详情): key y is visible from query x iff j_y = j_x,
// c_y in {0, c_x} and t_y <= t_x; a sliding-window layer also needs
// t_x - t_y < W.  Because the stream keeps every trunk and every question
// contiguous, the visible keys of a query row are at most three contiguous
// ranges, visited in this fixed order:
//   (A) the checkpointed prefix, positions 0..m-1, from the K/V cache slot of a
//       resumed request (Korean summary §어떻게 쓰나: K/V before m are kept);
//   (B) for a question row, every trunk row of its request (all positions < P);
//   (C) the rows of the query's own segment up to and including itself.
// Windowing only trims the front of this list.  The order depends only on the
// request, never on the rest of the round, so every output bit is independent
// of the round's composition.
#include "device_common.hpp"

namespace flide {

// ---------------------------------------------------------------------------
// Plain kernel: one wave per (query row, q head); lane-per-key scores.
// Used for fp32 mode and any head size the MFMA kernel does not cover.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) attn_plain_kernel(MetaView mv, const T* __restrict__ q,
                                                         const T* __restrict__ k_rot, const T* __restrict__ v,
                                                         const T* __restrict__ k_cache,
                                                         const T* __restrict__ v_cache, T* __restrict__ o,
                                                         const float* __restrict__ table, int max_pos, int Hq,
                                                         int Hkv, int d, int window, int cache_rows,
                                                         int cache_slots) {
  __shared__ float q_lds[4][256];
  const int tile = blockIdx.x;
  if (tile >= mv.hdr[H_NTILES]) return;
  const int h = blockIdx.y;
  const int g = h / (Hq / Hkv);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int s = mv.tile_seg[tile];
  if (s < 0 || s >= mv.hdr[H_NSEG]) {
    if (threadIdx.x == 0) flag_error(mv.dev_error, E_SEGMENT);
    return;
  }
  const int seg_row0 = mv.seg_row0[s], seg_len = mv.seg_len[s];
  const int j = mv.seg_req[s];
  const bool question = mv.seg_branch[s] > 0;
  const int P = mv.req_P[j], m = mv.req_m[j];
  if (m > 0 && (m > cache_rows || k_cache == nullptr || mv.req_ckpt[j] < 0 || mv.req_ckpt[j] >= cache_slots)) {
    if (threadIdx.x == 0) flag_error(mv.dev_error, E_CACHE);
    return;
  }
  const int ckpt = mv.req_ckpt[j];
  const float scale = rsqrtf(float(d));
  const int half = d >> 1;
  const int per_lane = (d + 63) / 64;

  for (int r = wave; r < kTileRows; r += 4) {
    const int x = mv.tile_row0[tile] + r;
    if (x >= seg_row0 + seg_len) break;
    const int tx = mv.seg_pos0[s] + (x - seg_row0);
    if (tx >= max_pos) {
      if (lane == 0) flag_error(mv.dev_error, E_POSITION);
      continue;
    }
    // rotated query into LDS
    const int64_t qb = (int64_t(x) * Hq + h) * d;
    for (int e = lane; e < half; e += 64) {
      float c = table[(int64_t(tx) * half + e) * 2], sn = table[(int64_t(tx) * half + e) * 2 + 1];
      float x1 = load_f32(q, qb + e), x2 = load_f32(q, qb + e + half);
      q_lds[wave][e] = x1 * c - x2 * sn;
      q_lds[wave][e + half] = x2 * c + x1 * sn;
    }
    __builtin_amdgcn_wave_barrier();
    const int lo_pos = window > 0 ? tx - window + 1 : 0;
    float mrun = -INFINITY, lrun = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};

    // key source k: 0 = cache, 1 = trunk rows, 2 = own rows
    for (int src = 0; src < 3; ++src) {
      int n_keys = 0, first_pos = 0;
      const T* kp = nullptr;
      const T* vp = nullptr;
      int64_t row_stride = int64_t(Hkv) * d;
      int64_t base = 0;
      if (src == 0) {
        if (m == 0) continue;
        int lo = max(lo_pos, 0);
        n_keys = m - lo;
        first_pos = lo;
        kp = k_cache;
        vp = v_cache;
        base = ((int64_t(ckpt) * cache_rows + lo) * Hkv + g) * d;
      } else if (src == 1) {
        if (!question) continue;
        int trow0 = mv.req_trunk_row0[j];
        int lo = max(lo_pos, m);
        n_keys = P - lo;
        first_pos = lo;
        kp = k_rot;
        vp = v;
        base = ((int64_t(trow0) + (lo - m)) * Hkv + g) * d;
      } else {
        int pos0 = mv.seg_pos0[s];
        int lo = max(lo_pos, pos0);
        n_keys = tx - lo + 1;
        first_pos = lo;
        kp = k_rot;
        vp = v;
        base = ((int64_t(seg_row0) + (lo - pos0)) * Hkv + g) * d;
      }
      (void)first_pos;
      for (int kb = 0; kb < n_keys; kb += 64) {
        const int key = kb + lane;
        float sc = -INFINITY;
        if (key < n_keys) {
          const int64_t kr = base + int64_t(key) * row_stride;
          float acc_s = 0.f;
          for (int e = 0; e < d; ++e) acc_s += q_lds[wave][e] * load_f32(kp, kr + e);
          sc = acc_s * scale;
        }
        const float mblk = wave_max(sc);
        const float mnew = fmaxf(mrun, mblk);
        const float corr = (mrun == -INFINITY) ? 0.f : __expf(mrun - mnew);
        const float p = (key < n_keys) ? __expf(sc - mnew) : 0.f;
        lrun = lrun * corr + wave_sum(p);
        mrun = mnew;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= corr;
        const int nb = min(64, n_keys - kb);
        for (int kk = 0; kk < nb; ++kk) {
          const float pk = __shfl(p, kk, 64);
          const int64_t vr = base + int64_t(kb + kk) * row_stride;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            if (i < per_lane && e < d) acc[i] += pk * load_f32(vp, vr + e);
          }
        }
      }
    }
    const float inv = 1.f / lrun;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (i < per_lane && e < d) store_f32(o, qb + e, acc[i] * inv);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

int launch_attn(const MetaView& mv, const flide_attn_params& p, const RopeArgs& rope, const void* q,
                const void* k_rot, const void* v, const void* k_cache, const void* v_cache, void* o,
                void* stream) {
  dim3 grid(mv.tile_cap, p.Hq);
  int W = p.window;
  if (p.dtype == FLIDE_BF16) {
    hipLaunchKernelGGL(attn_plain_kernel<bf16_t>, grid, dim3(256), 0, (hipStream_t)stream, mv, (const bf16_t*)q,
                       (const bf16_t*)k_rot, (const bf16_t*)v, (const bf16_t*)k_cache, (const bf16_t*)v_cache,
                       (bf16_t*)o, rope.table, rope.max_pos, p.Hq, p.Hkv, p.d, W, p.cache_rows, p.cache_slots);
  } else {
    hipLaunchKernelGGL(attn_plain_kernel<float>, grid, dim3(256), 0, (hipStream_t)stream, mv, (const float*)q,
                       (const float*)k_rot, (const float*)v, (const float*)k_cache, (const float*)v_cache,
                       (float*)o, rope.table, rope.max_pos, p.Hq, p.Hkv, p.d, W, p.cache_rows, p.cache_slots);
  }
  return int(hipGetLastError());
}

}  // namespace flide
