// Metadata expansion and key rotation.
//
// meta_expand turns the uploaded segment table into per-row (j, c, t) labels
// ("Flide: Accelerating Decision Inference with Exact State Forking"
// §方法步骤详情: every token carries request, branch and position; question
// positions continue from P), marks tail rows (-1, -1, -1) (Korean summary
// §어떻게 쓰나: padding only at the tail), and writes one descriptor per
// attention work-list position (tile_desc), so that an attention workgroup
// reads its units, request and key ranges from one record.
//
// rope_k rotates every key row once to its metadata position (rotate-half
// pairs (i, i + d/2), angle t * theta^(-2i/d), host fp64 table stored fp32), so
// the attention kernel's inner loop reads rotated keys directly.
#include "device_common.hpp"

namespace flide {

__global__ void __launch_bounds__(256) meta_expand_kernel(MetaView mv) {
  const int T = mv.hdr[H_T];
  const int n_seg = mv.hdr[H_NSEG];
  const bool bad = mv.hdr[H_MAGIC] != kMagic || T < 0 || T > mv.T_cap || n_seg < 0 || n_seg > mv.seg_cap ||
                   mv.hdr[H_R] < 0 || mv.hdr[H_R] > mv.R_cap || mv.hdr[H_NQST] < 0 ||
                   mv.hdr[H_NQST] > mv.Q_cap || mv.hdr[H_NTILES] < 0 || mv.hdr[H_NTILES] > mv.tile_cap;
  const int stride = gridDim.x * blockDim.x;
  // attention work-list descriptors: everything a tile's workgroup needs, in one record
  const int n_tiles = bad ? 0 : mv.hdr[H_NTILES];
  for (int x = blockIdx.x * blockDim.x + threadIdx.x; x < mv.tile_cap; x += stride) {
    int32_t d[kTileDescWords];
#pragma unroll
    for (int i = 0; i < kTileDescWords; ++i) d[i] = 0;
    d[TD_SEG] = -1;
    const int s0 = x < n_tiles ? mv.tile_seg[int64_t(x) * kTileUnits] : -1;
    if (s0 >= 0 && s0 < n_seg) {
      const int j = mv.seg_req[s0];
      bool ok = true;
      int own_seg[kTileUnits];
      int nown = 0, qmin = INT_MAX, qmax = INT_MIN;
#pragma unroll
      for (int u = 0; u < kTileUnits; ++u) {
        const int s = mv.tile_seg[int64_t(x) * kTileUnits + u];
        if (s < 0) continue;
        if (s >= n_seg || mv.seg_req[s] != j) {
          ok = false;
          continue;
        }
        const int row0 = mv.seg_row0[s], pos0 = mv.seg_pos0[s];
        const int x0 = mv.tile_row0[int64_t(x) * kTileUnits + u];
        const int nr = min(kUnitRows, row0 + mv.seg_len[s] - x0);
        if (x0 < row0 || nr <= 0) {
          ok = false;
          continue;
        }
        int k = 0;
        while (k < nown && own_seg[k] != s) ++k;
        if (k == nown) {
          own_seg[nown++] = s;
          d[TD_OWN + 4 * k + TO_ROFF] = row0 - pos0;
          d[TD_OWN + 4 * k + TO_VOFF] = mv.seg_vcol0[s];
          d[TD_OWN + 4 * k + TO_LO] = pos0;
        }
        const int q0 = pos0 + (x0 - row0);
        d[TD_OWN + 4 * k + TO_HI] = max(d[TD_OWN + 4 * k + TO_HI], q0 + nr);
        d[TD_UNIT + 4 * u + TU_ROW0] = x0;
        d[TD_UNIT + 4 * u + TU_NROWS] = nr;
        d[TD_UNIT + 4 * u + TU_QPOS0] = q0;
        d[TD_UNIT + 4 * u + TU_OWN] = k;
        qmin = min(qmin, q0);
        qmax = max(qmax, q0 + nr - 1);
      }
      if (ok) {
        d[TD_SEG] = s0;
        d[TD_QUESTION] = mv.seg_branch[s0] > 0 ? 1 : 0;
        d[TD_P] = mv.req_P[j];
        d[TD_M] = mv.req_m[j];
        d[TD_CKPT] = mv.req_ckpt[j];
        d[TD_ROFF_TRUNK] = mv.req_trunk_row0[j] - mv.req_m[j];
        d[TD_VOFF_TRUNK] = mv.seg_vcol0[j];  // the trunk segment of request j is segment j
        d[TD_QPOS_MIN] = qmin;
        d[TD_QPOS_MAX] = qmax;
        d[TD_NOWN] = nown;
      } else {
        flag_error(mv.dev_error, E_SEGMENT);
      }
    } else if (s0 != -1) {
      flag_error(mv.dev_error, E_SEGMENT);
    }
    int4* dst = reinterpret_cast<int4*>(mv.tile_desc + int64_t(x) * kTileDescWords);
#pragma unroll
    for (int i = 0; i < kTileDescWords / 4; ++i) dst[i] = int4{d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]};
  }
  if (bad) {
    if (blockIdx.x == 0 && threadIdx.x == 0) flag_error(mv.dev_error, E_HEADER);
    for (int row = blockIdx.x * blockDim.x + threadIdx.x; row < mv.T_cap; row += stride) {
      mv.tok_j[row] = -1;
      mv.tok_c[row] = -1;
      mv.tok_t[row] = -1;
    }
    return;
  }
  for (int row = blockIdx.x * blockDim.x + threadIdx.x; row < mv.T_cap; row += stride) {
    int j = -1, c = -1, t = -1;
    if (row < T && n_seg > 0) {
      int s = find_segment(mv.seg_row0, n_seg, row);
      int off = row - mv.seg_row0[s];
      if (off >= 0 && off < mv.seg_len[s]) {
        j = mv.seg_req[s];
        c = mv.seg_branch[s];
        t = mv.seg_pos0[s] + off;
      } else if (threadIdx.x == 0) {
        flag_error(mv.dev_error, E_SEGMENT);
      }
    }
    mv.tok_j[row] = j;
    mv.tok_c[row] = c;
    mv.tok_t[row] = t;
  }
}

__global__ void clear_error_kernel(int32_t* dev_error) {
  if (threadIdx.x < 4) dev_error[threadIdx.x] = 0;
}

int launch_meta_expand(const MetaView& mv, void* stream) {
  int blocks = (max(mv.T_cap, mv.tile_cap) + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(meta_expand_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, mv);
  return int(hipGetLastError());
}

int launch_clear_error(const MetaView& mv, void* stream) {
  hipLaunchKernelGGL(clear_error_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, mv.dev_error);
  return int(hipGetLastError());
}

// One thread rotates 4 consecutive pairs of one (row, kv head).
template <typename T>
__global__ void __launch_bounds__(256) rope_k_kernel(MetaView mv, const T* __restrict__ k, T* __restrict__ k_rot,
                                                     const float* __restrict__ table, int max_pos, int Hkv,
                                                     int d) {
  const int T_rows = mv.hdr[H_T];
  const int half = d >> 1;
  const int groups = half >> 2;  // 4 pairs per thread
  const int64_t per_row = int64_t(Hkv) * groups;
  const int64_t total = int64_t(T_rows) * per_row;
  for (int64_t w = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; w < total;
       w += int64_t(gridDim.x) * blockDim.x) {
    const int row = int(w / per_row);
    const int rem = int(w - int64_t(row) * per_row);
    const int h = rem / groups;
    const int i0 = (rem - h * groups) * 4;
    const int pos = mv.tok_t[row];
    const int64_t base = (int64_t(row) * Hkv + h) * d;
    if (pos < 0 || pos >= max_pos) {
      if (pos >= max_pos) flag_error(mv.dev_error, E_POSITION);
      continue;
    }
    const float* cs = table + (int64_t(pos) * half + i0) * 2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float c = cs[2 * e], s = cs[2 * e + 1];
      float x1 = load_f32(k, base + i0 + e);
      float x2 = load_f32(k, base + i0 + e + half);
      store_f32(k_rot, base + i0 + e, x1 * c - x2 * s);
      store_f32(k_rot, base + i0 + e + half, x2 * c + x1 * s);
    }
  }
}

int launch_rope_k(const MetaView& mv, const flide_attn_params& p, const RopeArgs& rope, const void* k,
                  void* k_rot, void* stream) {
  int64_t work = int64_t(mv.T_cap) * p.Hkv * (p.d / 8);
  int blocks = int((work + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  if (p.dtype == FLIDE_BF16)
    hipLaunchKernelGGL(rope_k_kernel<bf16_t>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, mv,
                       (const bf16_t*)k, (bf16_t*)k_rot, rope.table, rope.max_pos, p.Hkv, p.d);
  else
    hipLaunchKernelGGL(rope_k_kernel<float>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, mv,
                       (const float*)k, (float*)k_rot, rope.table, rope.max_pos, p.Hkv, p.d);
  return int(hipGetLastError());
}

}  // namespace flide
