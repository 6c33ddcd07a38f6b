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
// Windowing only trims the front of this list.  Key tiles are aligned in
// position space (multiples of the tile size), so the grouping of keys — and
// therefore every rounding step of the online softmax — depends only on the
// request, never on the rest of the round: outputs are bit-identical whatever
// the round's composition.
#include "device_common.hpp"

namespace flide {

// ---------------------------------------------------------------------------
// Plain kernel: one wave per (query row, q head); lane-per-key scores.
// Used for fp32 mode and head sizes the MFMA kernel does not cover.
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
  const int ckpt = mv.req_ckpt[j];
  if (m > 0 && (m > cache_rows || k_cache == nullptr || ckpt < 0 || ckpt >= cache_slots)) {
    if (threadIdx.x == 0) flag_error(mv.dev_error, E_CACHE);
    return;
  }
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

    for (int src = 0; src < 3; ++src) {
      int n_keys = 0;
      const T* kp = nullptr;
      int64_t kbase = 0;            // element offset of the first key row (kv head g)
      const int64_t kstride = int64_t(Hkv) * d;
      // values: element (key, e) at vp[vbase + key * vkey + e * ve]
      const T* vp = nullptr;
      int64_t vbase = 0, vkey = 0, ve = 1;
      if (src == 0) {
        if (m == 0) continue;
        const int lo = max(lo_pos, 0);
        n_keys = m - lo;
        kp = k_cache;
        kbase = ((int64_t(ckpt) * cache_rows + lo) * Hkv + g) * d;
        vp = v_cache;  // [slot, Hkv, d, cache_rows]
        vbase = (int64_t(ckpt) * Hkv + g) * d * cache_rows + lo;
        vkey = 1;
        ve = cache_rows;
      } else if (src == 1) {
        if (!question) continue;
        const int lo = max(lo_pos, m);
        n_keys = P - lo;
        const int64_t row = int64_t(mv.req_trunk_row0[j]) + (lo - m);
        kp = k_rot;
        kbase = (row * Hkv + g) * d;
        vp = v;
        vbase = kbase;
        vkey = kstride;
      } else {
        const int pos0 = mv.seg_pos0[s];
        const int lo = max(lo_pos, pos0);
        n_keys = tx - lo + 1;
        const int64_t row = int64_t(seg_row0) + (lo - pos0);
        kp = k_rot;
        kbase = (row * Hkv + g) * d;
        vp = v;
        vbase = kbase;
        vkey = kstride;
      }
      for (int kb = 0; kb < n_keys; kb += 64) {
        const int key = kb + lane;
        float sc = -INFINITY;
        if (key < n_keys) {
          const int64_t kr = kbase + int64_t(key) * kstride;
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
          const int64_t vr = vbase + int64_t(kb + kk) * vkey;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            if (i < per_lane && e < d) acc[i] += pk * load_f32(vp, vr + int64_t(e) * ve);
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

// ---------------------------------------------------------------------------
// MFMA path (bf16, d = 128 or 256)
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// D = A * B + C for a 16x16 tile with K = 32 (bf16 operands, fp32 accumulate).
// Lane l supplies A[l % 16][8 (l / 16) .. +7] and B[8 (l / 16) .. +7][l % 16] and
// receives C[4 (l / 16) + i][l % 16], i = 0..3.
__device__ __forceinline__ f32x4v mfma16x16x32(u32x4v a, u32x4v b, f32x4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a), __builtin_bit_cast(bf16x8v, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// Rows of the transposed value workspace per (kv head, channel): the stream
// capacity rounded up, plus room for one aligned over-read.
__host__ __device__ __forceinline__ int64_t vt_rows(int T_cap) { return ((int64_t(T_cap) + 63) / 64) * 64 + 64; }

// Prep pass of the MFMA path: rotate every key row once (rotate-half pairs at
// the row's metadata position) into k_rot [T_cap, Hkv, D], and write the values
// transposed into vt [Hkv, D, vt_rows] so value tiles load as contiguous rows.
template <int D>
__global__ void __launch_bounds__(256) kv_prep_kernel(MetaView mv, const bf16_t* __restrict__ k,
                                                      const bf16_t* __restrict__ v, bf16_t* __restrict__ k_rot,
                                                      bf16_t* __restrict__ vt, const float* __restrict__ table,
                                                      int max_pos, int Hkv) {
  constexpr int ROWS = 64;
  constexpr int STR = D + 2;
  __shared__ bf16_t v_lds[ROWS * STR];
  const int r0 = blockIdx.x * ROWS;
  const int g = blockIdx.y;
  const int T = mv.hdr[H_T];
  if (r0 >= mv.T_cap) return;
  const int tid = threadIdx.x;
  constexpr int HALF = D / 2;
  constexpr int GROUPS = HALF / 8;  // 8 pairs per work item
  // keys: rotate
  for (int it = tid; it < ROWS * GROUPS; it += 256) {
    const int rr = it / GROUPS, i0 = (it % GROUPS) * 8;
    const int row = r0 + rr;
    if (row >= T) continue;
    const int pos = mv.tok_t[row];
    if (pos < 0 || pos >= max_pos) {
      if (pos >= max_pos) flag_error(mv.dev_error, E_POSITION);
      continue;
    }
    const int64_t base = (int64_t(row) * Hkv + g) * D;
    const u32x4v a = *reinterpret_cast<const u32x4v*>(k + base + i0);
    const u32x4v b = *reinterpret_cast<const u32x4v*>(k + base + i0 + HALF);
    const float* cs = table + (int64_t(pos) * HALF + i0) * 2;
    u32x4v lo, hi;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float a0 = __uint_as_float(a[w] << 16), a1 = __uint_as_float(a[w] & 0xFFFF0000u);
      float b0 = __uint_as_float(b[w] << 16), b1 = __uint_as_float(b[w] & 0xFFFF0000u);
      float c0 = cs[4 * w], s0 = cs[4 * w + 1], c1 = cs[4 * w + 2], s1 = cs[4 * w + 3];
      lo[w] = pack_bf16x2(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
      hi[w] = pack_bf16x2(b0 * c0 + a0 * s0, b1 * c1 + a1 * s1);
    }
    *reinterpret_cast<u32x4v*>(k_rot + base + i0) = lo;
    *reinterpret_cast<u32x4v*>(k_rot + base + i0 + HALF) = hi;
  }
  // values: stage rows in LDS, write transposed (rows >= T become zeros)
  for (int it = tid; it < ROWS * (D / 8); it += 256) {
    const int rr = it / (D / 8), ch = it % (D / 8);
    const int row = r0 + rr;
    u32x4v val = {0u, 0u, 0u, 0u};
    if (row < T) val = *reinterpret_cast<const u32x4v*>(v + (int64_t(row) * Hkv + g) * D + ch * 8);
    uint32_t* dst = reinterpret_cast<uint32_t*>(v_lds + rr * STR + ch * 8);
    dst[0] = val[0];
    dst[1] = val[1];
    dst[2] = val[2];
    dst[3] = val[3];
  }
  __syncthreads();
  const int64_t VT = vt_rows(mv.T_cap);
  for (int it = tid; it < D * (ROWS / 8); it += 256) {
    const int c = it % (ROWS / 8), dd = it / (ROWS / 8);
    u32x4v out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t e0 = v_lds[(8 * c + 2 * w) * STR + dd];
      const uint32_t e1 = v_lds[(8 * c + 2 * w + 1) * STR + dd];
      out[w] = e0 | (e1 << 16);
    }
    *reinterpret_cast<u32x4v*>(vt + (int64_t(g) * D + dd) * VT + r0 + 8 * c) = out;
  }
}

// 8 consecutive bf16 starting at element `e` of a row whose 16-byte chunks are
// aligned; `o` = e & 7 is the same for every chunk of a key range.
__device__ __forceinline__ u32x4v load8_realign(const bf16_t* __restrict__ base, int64_t e, int o) {
  const bf16_t* a = base + (e - o);
  const u32x4v w0 = *reinterpret_cast<const u32x4v*>(a);
  if (o == 0) return w0;
  const u32x4v w1 = *reinterpret_cast<const u32x4v*>(a + 8);
  const uint32_t w[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
  const int dw = o >> 1;
  u32x4v r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t lo = w[k], hi = w[k + 1];
    if (dw == 1) { lo = w[k + 1]; hi = w[k + 2]; }
    if (dw == 2) { lo = w[k + 2]; hi = w[k + 3]; }
    if (dw == 3) { lo = w[k + 3]; hi = w[k + 4]; }
    r[k] = (o & 1) ? __builtin_amdgcn_alignbyte(hi, lo, 2) : lo;
  }
  return r;
}

// One workgroup = one query tile (32 rows of one segment) x up to 4 q heads of
// one kv head; wave w owns q head (group * 4 + w).  Scores are computed
// transposed (S^T = K Q^T: keys on MFMA rows, queries on columns) so that each
// lane holds whole query columns: softmax statistics and the rescale of the
// output accumulator (O^T = V^T P^T, d on rows) stay lane-local.
template <int D, int BN>
__global__ void __launch_bounds__(256) attn_mfma_kernel(MetaView mv, const bf16_t* __restrict__ q,
                                                        const bf16_t* __restrict__ k_rot,
                                                        const bf16_t* __restrict__ vt,
                                                        const bf16_t* __restrict__ k_cache,
                                                        const bf16_t* __restrict__ v_cache, bf16_t* __restrict__ o,
                                                        const float* __restrict__ table, int max_pos, int Hq,
                                                        int Hkv, int window, int cache_rows, int cache_slots) {
  constexpr int NC = D / 32;   // 32-wide d chunks of the score contraction
  constexpr int NDB = D / 16;  // 16-wide d blocks of the output
  constexpr int NKB = BN / 16; // 16-key blocks per tile
  constexpr int KSTR = D + 8;  // LDS row stride of the key tile (elements)
  constexpr int VSTR = BN + 4; // LDS row stride of the transposed value tile (elements)
  __shared__ __attribute__((aligned(16))) bf16_t k_lds[BN * KSTR];
  __shared__ __attribute__((aligned(16))) bf16_t v_lds[D * VSTR];

  const int tile = blockIdx.x;
  if (tile >= mv.hdr[H_NTILES]) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g4 = l >> 4;
  const int G = Hq / Hkv;
  const int HG = (G + 3) / 4;
  const int kvh = blockIdx.y / HG, hl = (blockIdx.y % HG) * 4 + w;
  const bool active = hl < G;
  const int h = kvh * G + hl;

  const int seg = mv.tile_seg[tile];
  if (seg < 0 || seg >= mv.hdr[H_NSEG]) {
    if (tid == 0) flag_error(mv.dev_error, E_SEGMENT);
    return;
  }
  const int seg_row0 = mv.seg_row0[seg], seg_len = mv.seg_len[seg], pos0 = mv.seg_pos0[seg];
  const int j = mv.seg_req[seg];
  const bool question = mv.seg_branch[seg] > 0;
  const int P = mv.req_P[j], m = mv.req_m[j], ckpt = mv.req_ckpt[j];
  if (m > 0 && (m > cache_rows || k_cache == nullptr || ckpt < 0 || ckpt >= cache_slots)) {
    if (tid == 0) flag_error(mv.dev_error, E_CACHE);
    return;
  }
  const int x0 = mv.tile_row0[tile];
  const int nrows = min(kTileRows, seg_row0 + seg_len - x0);
  const int qpos_min = pos0 + (x0 - seg_row0);
  const int qpos_max = qpos_min + nrows - 1;
  if (qpos_max >= max_pos) {
    if (tid == 0) flag_error(mv.dev_error, E_POSITION);
    return;
  }

  // ---- rotated queries, as MFMA B fragments (query = column) ----
  u32x4v qf[2][NC];
  int qpos[2];
  bool qvalid[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = qb * 16 + r16;
    qvalid[qb] = active && r < nrows;
    qpos[qb] = qpos_min + r;
#pragma unroll
    for (int c = 0; c < NC / 2; ++c) {
      u32x4v lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      if (qvalid[qb]) {
        const int64_t base = (int64_t(x0 + r) * Hq + h) * D + 32 * c + 8 * g4;
        const u32x4v a = *reinterpret_cast<const u32x4v*>(q + base);
        const u32x4v b = *reinterpret_cast<const u32x4v*>(q + base + D / 2);
        const float* cs = table + (int64_t(qpos[qb]) * (D / 2) + 32 * c + 8 * g4) * 2;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          float a0 = __uint_as_float(a[ww] << 16), a1 = __uint_as_float(a[ww] & 0xFFFF0000u);
          float b0 = __uint_as_float(b[ww] << 16), b1 = __uint_as_float(b[ww] & 0xFFFF0000u);
          float c0 = cs[4 * ww], s0 = cs[4 * ww + 1], c1 = cs[4 * ww + 2], s1 = cs[4 * ww + 3];
          lo[ww] = pack_bf16x2(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
          hi[ww] = pack_bf16x2(b0 * c0 + a0 * s0, b1 * c1 + a1 * s1);
        }
      }
      qf[qb][c] = lo;
      qf[qb][c + NC / 2] = hi;
    }
  }

  f32x4v acc[2][NDB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x4v{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  const float sl2 = 1.4426950408889634f * rsqrtf(float(D));
  const int lo_w = window > 0 ? qpos_min - window + 1 : INT_MIN;
  const int64_t VT = vt_rows(mv.T_cap);

  for (int src = 0; src < 3; ++src) {
    // positions [lo, hi) of this key range; key row r(p) = p + roff
    int lo, hi;
    int64_t roff;
    const bf16_t* kptr;
    const bf16_t* vptr;
    int64_t vstride;
    if (src == 0) {
      if (m == 0) continue;
      lo = max(0, lo_w);
      hi = min(m, qpos_max + 1);
      roff = int64_t(ckpt) * cache_rows;
      kptr = k_cache + int64_t(kvh) * D;
      vptr = v_cache + (int64_t(ckpt) * Hkv + kvh) * D * cache_rows;
      vstride = cache_rows;
    } else if (src == 1) {
      if (!question) continue;
      lo = max(m, lo_w);
      hi = P;
      roff = int64_t(mv.req_trunk_row0[j]) - m;
      kptr = k_rot + int64_t(kvh) * D;
      vptr = vt + int64_t(kvh) * D * VT;
      vstride = VT;
    } else {
      lo = max(pos0, lo_w);
      hi = qpos_max + 1;
      roff = int64_t(seg_row0) - pos0;
      kptr = k_rot + int64_t(kvh) * D;
      vptr = vt + int64_t(kvh) * D * VT;
      vstride = VT;
    }
    if (lo >= hi) continue;
    const int64_t vro = src == 0 ? 0 : roff;  // value column of position p: p + vro
    const int valign = int((vro % 8 + 8) % 8);
    for (int ts = lo - ((lo % BN) + BN) % BN; ts < hi; ts += BN) {
      __syncthreads();
      // key tile [BN][D]
      for (int it = tid; it < BN * (D / 8); it += 256) {
        const int kk = it / (D / 8), ch = it % (D / 8);
        const int p = ts + kk;
        u32x4v val = {0u, 0u, 0u, 0u};
        if (p >= lo && p < hi)
          val = *reinterpret_cast<const u32x4v*>(kptr + (int64_t(p) + roff) * (int64_t(Hkv) * D) + ch * 8);
        *reinterpret_cast<u32x4v*>(k_lds + kk * KSTR + ch * 8) = val;
      }
      // transposed value tile [D][BN]
      for (int it = tid; it < D * (BN / 8); it += 256) {
        const int c = it % (BN / 8), dd = it / (BN / 8);
        const int p0 = ts + 8 * c;
        u32x4v val = {0u, 0u, 0u, 0u};
        const bf16_t* row = vptr + int64_t(dd) * vstride;
        if (p0 >= lo && p0 + 7 < hi) {
          val = load8_realign(row, int64_t(p0) + vro, valign);
        } else if (p0 + 7 >= lo && p0 < hi) {
          uint32_t e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int p = p0 + i;
            e[i] = (p >= lo && p < hi) ? uint32_t(row[int64_t(p) + vro]) : 0u;
          }
          val = u32x4v{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
        }
        u32x2v* dst = reinterpret_cast<u32x2v*>(v_lds + dd * VSTR + 8 * c);
        dst[0] = u32x2v{val[0], val[1]};
        dst[1] = u32x2v{val[2], val[3]};
      }
      __syncthreads();
      if (!active) continue;

      // S^T = K Q^T over the tile
      f32x4v s[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb][0] = f32x4v{0.f, 0.f, 0.f, 0.f};
        s[kb][1] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const u32x4v a = *reinterpret_cast<const u32x4v*>(k_lds + (kb * 16 + r16) * KSTR + 32 * c + 8 * g4);
          s[kb][0] = mfma16x16x32(a, qf[0][c], s[kb][0]);
          s[kb][1] = mfma16x16x32(a, qf[1][c], s[kb][1]);
        }
      }
      // mask, scale (log2 domain), online softmax per query column
      const bool full = ts >= lo && ts + BN <= hi && ts + BN - 1 <= qpos_min &&
                        (window == 0 || qpos_max - ts < window);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int p = ts + kb * 16 + 4 * g4 + i;
            const bool ok = full || (p >= lo && p < hi && p <= qpos[qb] && (window == 0 || qpos[qb] - p < window));
            const float v = ok ? s[kb][qb][i] * sl2 : -INFINITY;
            s[kb][qb][i] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run[qb], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float corr = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pv = __builtin_amdgcn_exp2f(s[kb][qb][i] - m_use);
            s[kb][qb][i] = pv;
            rs += pv;
          }
        rs += __shfl_xor(rs, 16, 64);
        rs += __shfl_xor(rs, 32, 64);
        l_run[qb] = l_run[qb] * corr + rs;
        m_run[qb] = m_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[qb][db] *= corr;
      }
      // O^T += V^T P^T: K-steps of 32 keys = key blocks (2 ks, 2 ks + 1)
#pragma unroll
      for (int ks = 0; ks < NKB / 2; ++ks) {
        u32x4v pf[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const f32x4v a = s[2 * ks][qb], b = s[2 * ks + 1][qb];
          pf[qb] = u32x4v{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                          pack_bf16x2(b[2], b[3])};
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16_t* vr = v_lds + (db * 16 + r16) * VSTR + 32 * ks + 4 * g4;
          const u32x2v x0v = *reinterpret_cast<const u32x2v*>(vr);
          const u32x2v x1v = *reinterpret_cast<const u32x2v*>(vr + 16);
          const u32x4v a = u32x4v{x0v[0], x0v[1], x1v[0], x1v[1]};
          acc[0][db] = mfma16x16x32(a, pf[0], acc[0][db]);
          acc[1][db] = mfma16x16x32(a, pf[1], acc[1][db]);
        }
      }
    }
  }

  if (!active) return;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (!qvalid[qb]) continue;
    const float inv = 1.f / l_run[qb];
    bf16_t* dst = o + (int64_t(x0 + qb * 16 + r16) * Hq + h) * D + 4 * g4;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const f32x4v a = acc[qb][db];
      *reinterpret_cast<u32x2v*>(dst + db * 16) =
          u32x2v{pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv)};
    }
  }
}

bool attn_uses_mfma(const flide_attn_params& p) { return p.dtype == FLIDE_BF16 && (p.d == 256 || p.d == 128); }

int64_t attn_workspace_bytes(const flide_caps& c, const flide_attn_params& p) {
  const int64_t elem = p.dtype == FLIDE_BF16 ? 2 : 4;
  int64_t bytes = int64_t(c.T_cap) * p.Hkv * p.d * elem;  // rotated keys
  if (attn_uses_mfma(p)) bytes += int64_t(p.Hkv) * p.d * vt_rows(c.T_cap) * elem;  // transposed values
  return bytes;
}

int launch_attn(const MetaView& mv, const flide_attn_params& p, const RopeArgs& rope, const void* q, const void* k,
                const void* v, const void* k_cache, const void* v_cache, void* o, void* workspace, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int W = p.window;
  if (attn_uses_mfma(p)) {
    bf16_t* k_rot = (bf16_t*)workspace;
    bf16_t* vt = k_rot + int64_t(mv.T_cap) * p.Hkv * p.d;
    dim3 pg((mv.T_cap + 63) / 64, p.Hkv);
    const int G = p.Hq / p.Hkv;
    dim3 grid(mv.tile_cap, p.Hkv * ((G + 3) / 4));
    if (p.d == 256) {
      hipLaunchKernelGGL(kv_prep_kernel<256>, pg, dim3(256), 0, st, mv, (const bf16_t*)k, (const bf16_t*)v, k_rot,
                         vt, rope.table, rope.max_pos, p.Hkv);
      hipLaunchKernelGGL((attn_mfma_kernel<256, 64>), grid, dim3(256), 0, st, mv, (const bf16_t*)q, k_rot, vt,
                         (const bf16_t*)k_cache, (const bf16_t*)v_cache, (bf16_t*)o, rope.table, rope.max_pos, p.Hq,
                         p.Hkv, W, p.cache_rows, p.cache_slots);
    } else {
      hipLaunchKernelGGL(kv_prep_kernel<128>, pg, dim3(256), 0, st, mv, (const bf16_t*)k, (const bf16_t*)v, k_rot,
                         vt, rope.table, rope.max_pos, p.Hkv);
      hipLaunchKernelGGL((attn_mfma_kernel<128, 64>), grid, dim3(256), 0, st, mv, (const bf16_t*)q, k_rot, vt,
                         (const bf16_t*)k_cache, (const bf16_t*)v_cache, (bf16_t*)o, rope.table, rope.max_pos, p.Hq,
                         p.Hkv, W, p.cache_rows, p.cache_slots);
    }
    return int(hipGetLastError());
  }
  int rc = launch_rope_k(mv, p, rope, k, workspace, stream);
  if (rc != 0) return rc;
  dim3 grid(mv.tile_cap, p.Hq);
  if (p.dtype == FLIDE_BF16) {
    hipLaunchKernelGGL(attn_plain_kernel<bf16_t>, grid, dim3(256), 0, st, mv, (const bf16_t*)q,
                       (const bf16_t*)workspace, (const bf16_t*)v, (const bf16_t*)k_cache, (const bf16_t*)v_cache,
                       (bf16_t*)o, rope.table, rope.max_pos, p.Hq, p.Hkv, p.d, W, p.cache_rows, p.cache_slots);
  } else {
    hipLaunchKernelGGL(attn_plain_kernel<float>, grid, dim3(256), 0, st, mv, (const float*)q,
                       (const float*)workspace, (const float*)v, (const float*)k_cache, (const float*)v_cache,
                       (float*)o, rope.table, rope.max_pos, p.Hq, p.Hkv, p.d, W, p.cache_rows, p.cache_slots);
  }
  return int(hipGetLastError());
}

}  // namespace flide
