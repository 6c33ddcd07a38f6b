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
#include <type_traits>

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
  const int s0 = mv.tile_seg[int64_t(tile) * kTileUnits];
  if (s0 == -1) return;  // unused position of the work list
  if (s0 < 0 || s0 >= mv.hdr[H_NSEG]) {
    if (threadIdx.x == 0) flag_error(mv.dev_error, E_SEGMENT);
    return;
  }
  const int j = mv.seg_req[s0];
  const int P = mv.req_P[j], m = mv.req_m[j];
  const int ckpt = mv.req_ckpt[j];
  if (m > 0 && (m > cache_rows || k_cache == nullptr || ckpt < 0 || ckpt >= cache_slots)) {
    if (threadIdx.x == 0) flag_error(mv.dev_error, E_CACHE);
    return;
  }
  const float scale = rsqrtf(float(d));
  const int half = d >> 1;
  const int per_lane = (d + 63) / 64;

  // row r of the tile: row r % kUnitRows of unit r / kUnitRows (the units' segments were checked by
  // meta_expand: one request, rows inside the segment)
  for (int r = wave; r < kTileRows; r += 4) {
    const int s = mv.tile_seg[int64_t(tile) * kTileUnits + r / kUnitRows];
    if (s < 0 || s >= mv.hdr[H_NSEG] || mv.seg_req[s] != j) continue;
    const int seg_row0 = mv.seg_row0[s], seg_len = mv.seg_len[s];
    const bool question = mv.seg_branch[s] > 0;
    const int x = mv.tile_row0[int64_t(tile) * kTileUnits + r / kUnitRows] + r % kUnitRows;
    if (x < seg_row0 || x >= seg_row0 + seg_len) continue;
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

// Two floats to two bf16 (round to nearest even) in one hardware conversion.

// Columns of the transposed value workspace per (kv head, channel): the stream
// capacity plus up to 31 alignment columns per segment, rounded up to whole blocks.
__host__ __device__ __forceinline__ int64_t vt_cols(int T_cap, int seg_cap) {
  return ((int64_t(T_cap) + 32 * int64_t(seg_cap) + 64 + 63) / 64) * 64;
}
// Tile-major transposed values: vt [Hkv, vt_cols / 32, D, 32] -- column block b of kv head g holds, per
// channel, the 32 values of columns 32 b .. 32 b + 31 -- so the value tile of 32 positions is one
// contiguous D x 64-byte block.  Element index of (kv head g, channel dd, column col):
__host__ __device__ __forceinline__ int64_t vt_index(int g, int dd, int64_t col, int D, int64_t VT) {
  return ((int64_t(g) * (VT / 32) + (col >> 5)) * D + dd) * 32 + (col & 31);
}

// Prep pass of the MFMA path: rotate every key row once (rotate-half pairs at
// the row's metadata position) into k_rot [T_cap, Hkv, D], and write the values
// transposed and tile-major into vt (vt_index); the value of position p of segment s
// lands in column seg_vcol0[s] + p, so 32-aligned positions start a column block.
//
// One workgroup = 64 rows of one kv head.  Every load of a thread is issued before the first use
// (value rows, key rows and positions, then the rotation table rows at those positions), so a
// workgroup waits for two memory round trips instead of one per loop step.  Workgroup ids are laid
// out so that the Hkv workgroups of one row block sit eight apart: they run on the same XCD at about
// the same time and share the table rows through its L2.
template <int D>
__global__ void __launch_bounds__(256) kv_prep_kernel(MetaView mv, const bf16_t* __restrict__ k,
                                                      const bf16_t* __restrict__ v, bf16_t* __restrict__ k_rot,
                                                      bf16_t* __restrict__ vt, const float* __restrict__ table,
                                                      int max_pos, int Hkv) {
  constexpr int ROWS = 64;
  constexpr int STR = D + 2;
  constexpr int HALF = D / 2;
  constexpr int GROUPS = HALF / 8;             // 8 pairs per key work item
  constexpr int KIT = ROWS * GROUPS / 256;     // key work items per thread
  constexpr int VIT = ROWS * (D / 8) / 256;    // 16-byte value chunks per thread
  static_assert(KIT >= 1 && VIT >= 1, "64 rows over 256 threads");
  __shared__ bf16_t v_lds[ROWS * STR];
  const int i8 = blockIdx.x / kXcdClasses;
  const int rb = kXcdClasses * (i8 / Hkv) + int(blockIdx.x % kXcdClasses), g = i8 % Hkv;
  const int r0 = rb * ROWS;
  const int T = mv.hdr[H_T];
  if (r0 >= T) return;
  const int tid = threadIdx.x;

  u32x4v vv[VIT];
#pragma unroll
  for (int i = 0; i < VIT; ++i) {
    const int it = tid + 256 * i, rr = it / (D / 8), ch = it % (D / 8);
    const int row = min(r0 + rr, T - 1);
    vv[i] = *reinterpret_cast<const u32x4v*>(v + (int64_t(row) * Hkv + g) * D + ch * 8);
  }
  u32x4v ka[KIT], kb[KIT];
  int kpos[KIT];
#pragma unroll
  for (int i = 0; i < KIT; ++i) {
    const int it = tid + 256 * i, rr = it / GROUPS, i0 = (it % GROUPS) * 8;
    const int row = min(r0 + rr, T - 1);
    const int64_t base = (int64_t(row) * Hkv + g) * D;
    ka[i] = *reinterpret_cast<const u32x4v*>(k + base + i0);
    kb[i] = *reinterpret_cast<const u32x4v*>(k + base + i0 + HALF);
    kpos[i] = mv.tok_t[row];
  }
  float4 cs[KIT][4];
#pragma unroll
  for (int i = 0; i < KIT; ++i) {
    const int it = tid + 256 * i, i0 = (it % GROUPS) * 8;
    const int pos = kpos[i] < 0 ? 0 : (kpos[i] >= max_pos ? max_pos - 1 : kpos[i]);
    const float4* c4 = reinterpret_cast<const float4*>(table + (int64_t(pos) * HALF + i0) * 2);
#pragma unroll
    for (int w = 0; w < 4; ++w) cs[i][w] = c4[w];
  }
  // values -> LDS (rows past T hold a copy of row T - 1 and are never stored)
#pragma unroll
  for (int i = 0; i < VIT; ++i) {
    const int it = tid + 256 * i, rr = it / (D / 8), ch = it % (D / 8);
    uint32_t* dst = reinterpret_cast<uint32_t*>(v_lds + rr * STR + ch * 8);
    dst[0] = vv[i][0];
    dst[1] = vv[i][1];
    dst[2] = vv[i][2];
    dst[3] = vv[i][3];
  }
  // rotated keys
#pragma unroll
  for (int i = 0; i < KIT; ++i) {
    const int it = tid + 256 * i, rr = it / GROUPS, i0 = (it % GROUPS) * 8;
    const int row = r0 + rr;
    if (row >= T || kpos[i] < 0) continue;
    if (kpos[i] >= max_pos) {
      flag_error(mv.dev_error, E_POSITION);
      continue;
    }
    const int64_t base = (int64_t(row) * Hkv + g) * D;
    u32x4v lo, hi;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a0 = __uint_as_float(ka[i][w] << 16), a1 = __uint_as_float(ka[i][w] & 0xFFFF0000u);
      const float b0 = __uint_as_float(kb[i][w] << 16), b1 = __uint_as_float(kb[i][w] & 0xFFFF0000u);
      const float4 t4 = cs[i][w];  // (cos, sin) of two consecutive pairs
      lo[w] = pack_bf16x2(a0 * t4.x - b0 * t4.y, a1 * t4.z - b1 * t4.w);
      hi[w] = pack_bf16x2(b0 * t4.x + a0 * t4.y, b1 * t4.z + a1 * t4.w);
    }
    *reinterpret_cast<u32x4v*>(k_rot + base + i0) = lo;
    *reinterpret_cast<u32x4v*>(k_rot + base + i0 + HALF) = hi;
  }
  // the row's value column: trunk rows belong to segment j (one trunk segment per request, in request
  // order), question c of request j to segment req_q_seg0[j] + c - 1; column = seg_vcol0[s] + position
  const int lane = tid & 63, w = tid >> 6;
  const int row = r0 + lane;
  int64_t col = -1;
  if (row < T) {
    const int j = mv.tok_j[row], c = mv.tok_c[row], t = mv.tok_t[row];
    if (j >= 0 && t >= 0) col = int64_t(mv.seg_vcol0[c == 0 ? j : mv.req_q_seg0[j] + c - 1]) + t;
  }
  __syncthreads();
  if (col < 0) return;
  const int64_t VT = vt_cols(mv.T_cap, mv.seg_cap);
  bf16_t* dst = vt + vt_index(g, 0, col, D, VT);
  for (int dd = w; dd < D; dd += 4) dst[dd * 32] = v_lds[lane * STR + dd];
}

typedef __attribute__((address_space(3))) void* lds_vptr_t;
typedef __attribute__((address_space(1))) void* gbl_vptr_t;

// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes bytes [16 i, 16 i + 16) after `lds_base` (a wave-uniform address).
__device__ __forceinline__ void async_copy16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_vptr_t)(src), (lds_vptr_t)(lds_base), 16, 0, 0);
}

// MFMA operand read from LDS, written as inline asm so that the compiler does not track it.  The
// compiler models a direct-to-LDS copy (global_load_lds) as an access that may reach LDS through the
// flat path; while one is in flight it drains every LDS read (lgkmcnt(0)) before the first use of any
// of them, which exposes the full LDS latency at each wait.  Reads issued here are waited for
// explicitly: lds_wait<N>(r) returns once at most N LDS reads issued after r's are outstanding (LDS
// reads of a wave complete in issue order), and ties r's register to that wait, so nothing uses r
// before it.  OFF is the instruction's immediate byte offset.
template <int OFF>
__device__ __forceinline__ u32x4v lds_read16(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset field");
  u32x4v r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x4v& r) {
  static_assert(N >= 0 && N < 16, "lgkmcnt field");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(N));
}
// f(integral_constant<int, I>) for I = B .. E - 1, in order (compile-time indices for the reads above).
// acc + lo + hi of a pair of bf16 values (one dot-product instruction against (1, 1))
__device__ __forceinline__ float add_bf16_pair(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, pair), __builtin_bit_cast(bf16x2v, 0x3f803f80u),
                                         acc, false);
}
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// One workgroup = one query tile (32 rows of one segment) x up to 4 q heads of
// one kv head; wave w owns q head (group * 4 + w).  Scores are computed
// transposed (S^T = K Q^T: keys on MFMA rows, queries on columns) so that each
// lane holds whole query columns: softmax statistics and the rescale of the
// output accumulator (O^T = V^T P^T, d on rows) stay lane-local.
//
// Key and value tiles of 32 keys are double-buffered in LDS and filled by
// direct global-to-LDS copies issued one tile ahead, so memory latency overlaps
// the MFMA work; 64 KB of LDS per workgroup leaves room for two workgroups per
// CU.  Both tiles are stored with an XOR swizzle of their 16-byte chunks (key
// row r: chunk c at slot c ^ ksw(r); value row d: chunk c at slot c ^ vsw(d)),
// which makes the MFMA operand reads bank-conflict free.
// Score block kb row r is key 8 (r / 4) + 4 kb + r % 4, so each lane ends up
// with the probabilities of 8 consecutive keys: exactly the k-slots of its
// P^T fragment, whose matching V^T fragment is then one 16-byte read.
//
// Online softmax in the log2 domain (queries are pre-scaled by log2(e)/sqrt(d)),
// with a lazily moved running maximum: the output accumulator is rescaled only
// when a column's maximum grows by more than 8 (a factor of 256), which keeps
// every exponent <= 2^8 and the result exact up to rounding.
// Swizzle of the key tile's 16-byte chunks: distinct for the 16 rows one MFMA
// operand read touches (rows 8a + 4kb + b, a, b in 0..3).
__device__ __forceinline__ int ksw(int row) { return (row & 3) | (((row >> 3) & 3) << 2); }
// Swizzle of the value tile's chunks (rows of four 16-byte chunks).  Measured on gfx950: a 16-byte LDS read
// (ds_read_b128) serves the wave in four groups of 16 lanes, lane l in group (l / 16) ^ (bit 2 of l ^ bit 3
// of l), and a group takes one pass when its lanes hit 16 distinct 16-byte columns of a 256-byte bank row
// (equal addresses are broadcast).  The V^T operand read (lane l: row l % 16, chunk l / 16) therefore needs
// distinct chunk ^ swizzle over rows 4a + b, a = 0..3, after that lane regrouping; ((row >> 2) & 3) alone
// leaves two rows of each group on one column and halves the read rate.
__device__ __forceinline__ int vsw(int row) { return ((row >> 2) & 3) ^ (((row >> 2) ^ (row >> 3)) & 1); }

template <int D, bool G4>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_mfma_kernel(MetaView mv, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_rot,
                 const bf16_t* __restrict__ vt, const bf16_t* __restrict__ k_cache,
                 const bf16_t* __restrict__ v_cache, bf16_t* __restrict__ o, const float* __restrict__ table,
                 int max_pos, int Hq, int Hkv, int window, int cache_rows, int cache_slots) {
  constexpr int BN = 32;             // keys per tile
  constexpr int NC = D / 32;         // 32-wide d chunks of the score contraction
  constexpr int NDB = D / 16;        // 16-wide d blocks of the output
  constexpr int KROW = D * 2;        // bytes per key row
  constexpr int KCH = D / 8;         // 16-byte chunks per key row
  constexpr int VROW = BN * 2;       // bytes per value row (one channel, BN keys)
  constexpr int TILE_BYTES = BN * D * 2;
  constexpr int IPW = TILE_BYTES / 1024 / 4;  // copy instructions per wave per tile (per K or V)
  static_assert(IPW >= 1, "tile split over 4 waves");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * TILE_BYTES];  // K0 K1 V0 V1

  // Workgroup i runs on XCD i mod 8: XCD c takes the work-list positions c, c + 8, ... (the planner
  // puts each group of tiles that share keys on one of them).  By default every head group of a
  // position runs in turn (neighbouring workgroups share one query tile's keys); when the planner sets
  // a tile group n (rounds whose tiles see thousands of keys each), a run of n positions of the class
  // goes first for head group 0, then for head group 1, and so on, so that the workgroups resident on
  // an XCD at one time stream the same kv head's keys through its L2.
  const int tid = threadIdx.x, l = tid & 63, r16 = l & 15, g4 = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (scalar: LDS copy targets are uniform)
  const int G = Hq / Hkv;
  const int HG = (G + 3) / 4;
  const int HY = Hkv * HG;
  const int i8 = blockIdx.x / kXcdClasses;
  const int xcd = int(blockIdx.x % kXcdClasses);
  int tile = kXcdClasses * (i8 / HY) + xcd, yy = i8 % HY;
  // The classes are balanced by the cost of full attention (keys up to a tile's last row).  A windowed layer's
  // tiles see at most W + 31 keys each, so for it that balance does not hold: it takes the positions in the
  // planner's windowed order (tile_swa: the band order of the same tiles), the head groups of a position one
  // after another, on whichever XCD is free.
  if (window > 0) {
    tile = mv.tile_swa[int(blockIdx.x) / HY];  // the grid has tile_cap entries per head group
    yy = int(blockIdx.x) % HY;
    if (tile < 0 || tile >= mv.tile_cap) return;  // no position (the descriptor read below needs one)
  }

  // the position's descriptor (written by meta_expand): one 64-byte load instead of a chain of table
  // lookups.  The grid has tile_cap positions per head group, so the load is in bounds before the
  // position is known to be used; issuing it beside the header saves a round trip.
  constexpr int kHeadWords = 16;  // the tile's own words; units and own ranges are read where they are used
  int32_t td[kHeadWords];
  // The descriptor is read-only here (meta_expand wrote it before this launch) and the same for every lane:
  // it is read through the scalar path (constant address space), in batches with one wait.
  typedef const int32_t __attribute__((address_space(4)))* desc_ptr;
  auto desc_of = [&](int x) { return (desc_ptr)(uintptr_t)(mv.tile_desc + int64_t(x) * kTileDescWords); };
  auto load_desc = [&]() {
    const desc_ptr src = desc_of(tile);
#pragma unroll
    for (int i = 0; i < kHeadWords; ++i) td[i] = src[i];
  };
  load_desc();
  const int n_tiles_round = mv.hdr[H_NTILES];
  const int K8 = mv.tile_cap / kXcdClasses;  // positions per class
  const int tgroup = min(max(mv.hdr[H_TGROUP], 0), K8);
  if (tgroup > 0 && window == 0) {  // tile-group order: a bijection of the same (position, head group) pairs
    const int sb = i8 / (tgroup * HY), first = sb * tgroup, run = min(tgroup, K8 - first);
    const int rem = i8 - sb * tgroup * HY;
    tile = kXcdClasses * (first + rem % run) + xcd;
    yy = rem / run;
    load_desc();
  }
  if (tile >= n_tiles_round) return;
  const int kvh = yy / HG, hg0 = (yy % HG) * 4;  // kv head; first q head of the group in this workgroup
  // q heads of this workgroup (1 .. 4); G4: every head group has four (then wave w holds unit w)
  const int ng = G4 ? 4 : min(4, G - hg0);
  const int seg = td[TD_SEG];
  if (seg < 0) return;  // unused position (an inconsistent segment was flagged by meta_expand)
  const bool question = td[TD_QUESTION] != 0;
  const int P = td[TD_P], m = td[TD_M], ckpt = td[TD_CKPT];
  if (m > 0 && (m > cache_rows || k_cache == nullptr || ckpt < 0 || ckpt >= cache_slots)) {
    if (tid == 0) flag_error(mv.dev_error, E_CACHE);
    return;
  }
  const int qpos_min = td[TD_QPOS_MIN], qpos_max = td[TD_QPOS_MAX];
  const int n_own = min(td[TD_NOWN], kTileUnits);
  if (qpos_max >= max_pos) {
    if (tid == 0) flag_error(mv.dev_error, E_POSITION);
    return;
  }
  // Query columns: the tile's 32 rows x ng heads in row-major order, wave w taking columns 32 w .. 32 w + 31
  // (column k is row k / ng of head hg0 + k % ng; tile row r is row r % kUnitRows of unit r / kUnitRows,
  // whose rows belong to one segment: a trunk or one question).  All heads of a row see the same keys, and
  // each column's arithmetic involves that column only, so the assignment of columns to waves and lanes
  // changes no bit; with four heads a wave holds one unit, and a wave without a row (a short tile) skips
  // the key loop's arithmetic.
  // With four heads the wave's unit is w: its words are read once into scalars.  Otherwise a lane reads the
  // words of its row's unit from the record (a cached per-lane load).
  const desc_ptr unit_desc = desc_of(tile) + TD_UNIT;
  const int32_t* unit_vec = mv.tile_desc + int64_t(tile) * kTileDescWords + TD_UNIT;
  int w_row0 = 0, w_nrows = 0, w_qpos0 = 0, w_own = 0;
  if constexpr (G4) {
    const desc_ptr ud = unit_desc + 4 * w;
    w_row0 = ud[TU_ROW0], w_nrows = ud[TU_NROWS], w_qpos0 = ud[TU_QPOS0], w_own = ud[TU_OWN];
  }
  const desc_ptr own_desc = desc_of(tile) + TD_OWN;
  auto own_word = [&](int k, int f) __attribute__((always_inline)) { return own_desc[4 * k + f]; };
  struct ColInfo {
    bool valid;
    int row, pos, own;  // stream row, position and own key range of a valid column
  };
  // tile row r (column k is row k / ng); selects only, no branch that splits the wave (an invalid row reads
  // a valid stream row at a valid position)
  auto row_info = [&](int r) __attribute__((always_inline)) {
    // with four heads, the rows of wave w's columns (and of its share of the table rows) are unit w's
    const int ri = r % kUnitRows;
    int row0, nrows, qpos0, own;
    if constexpr (G4) {
      row0 = w_row0, nrows = w_nrows, qpos0 = w_qpos0, own = w_own;
    } else {
      const int32_t* ud = unit_vec + 4 * min(r / kUnitRows, kTileUnits - 1);
      row0 = ud[TU_ROW0], nrows = ud[TU_NROWS], qpos0 = ud[TU_QPOS0], own = ud[TU_OWN];
    }
    const bool valid = (r < kTileRows) & (ri < nrows);  // both evaluated: no branch
    return ColInfo{valid, valid ? row0 + ri : unit_desc[TU_ROW0], valid ? qpos0 + ri : qpos_min, own};
  };
  auto col_info = [&](int col) __attribute__((always_inline)) { return row_info(col / ng); };
  // this lane's two query columns (blocks qb = 0, 1): position and own key range, kept for the key loop
  int qpos[2], qown[2];
  bool active, qvalid[2];
  int own_mask = 0;  // own key ranges that some column of this wave reads (bit k: own range k)
  {
    const ColInfo c0 = col_info(32 * w + r16), c1 = col_info(32 * w + 16 + r16);
    qpos[0] = c0.pos, qpos[1] = c1.pos, qown[0] = c0.own, qown[1] = c1.own;
    qvalid[0] = c0.valid, qvalid[1] = c1.valid;
    active = __builtin_amdgcn_ballot_w64(c0.valid || c1.valid) != 0;
#pragma unroll
    for (int k = 0; k < kTileUnits; ++k)
      if (__builtin_amdgcn_ballot_w64((c0.valid && c0.own == k) || (c1.valid && c1.own == k))) own_mask |= 1 << k;
    own_mask = __builtin_amdgcn_readfirstlane(own_mask);
  }
  // the same flag as a scalar integer: tested once per key tile, where a boolean would be rebuilt from a
  // lane mask with vector instructions
  const int active_s = __builtin_amdgcn_readfirstlane(int(active));
  const int64_t VT = vt_cols(mv.T_cap, mv.seg_cap);
  const int lo_w = window > 0 ? qpos_min - window + 1 : INT_MIN;

  // ---- the key ranges: positions [lo, hi), key row = p + roff, value column = p + voff ----
  // (A) checkpoint cache, (B) the request's trunk rows (question tiles only), (C_k) own rows: one range per
  // segment among the tile's units (a trunk, or each question of a packed tile), read only by its columns
  const int lo0 = max(0, lo_w), hi0 = m > 0 ? min(m, qpos_max + 1) : 0;
  const int lo1 = max(m, lo_w), hi1 = question ? P : 0;
  const int64_t roff0 = int64_t(ckpt) * cache_rows, roff1 = td[TD_ROFF_TRUNK];
  const int64_t voff1 = td[TD_VOFF_TRUNK];
  const int ts00 = lo0 & ~(BN - 1), ts01 = lo1 & ~(BN - 1);
  const int n0 = lo0 < hi0 ? (hi0 - ts00 + BN - 1) / BN : 0;
  const int n1 = lo1 < hi1 ? (hi1 - ts01 + BN - 1) / BN : 0;
  int n_tiles = n0 + n1;
  {
    int olo[kTileUnits], ohi[kTileUnits];  // read together (one scalar round trip), unused ranges ignored
#pragma unroll
    for (int k = 0; k < kTileUnits; ++k) olo[k] = own_word(k, TO_LO), ohi[k] = own_word(k, TO_HI);
#pragma unroll
    for (int k = 0; k < kTileUnits; ++k) {  // an own range holds its units' positions, so it is never empty
      const int lo = max(olo[k], lo_w), hi = ohi[k];
      if (k < n_own) n_tiles += lo < hi ? (hi - (lo & ~(BN - 1)) + BN - 1) / BN : 0;
    }
  }
  // A cursor walks the key tiles in order: range rg (0 = A, 1 = B, 2 + k = C_k), tile start ts (a position) and the
  // byte addresses of the tile's first key row (kp) and of the first value column of this wave's first
  // value row (vp), advanced by one tile's stride (vstep for values); vrow is the byte stride of value
  // rows: the checkpoint cache holds whole transposed rows, the workspace one 64-byte row per block.  The range's
  // parameters are looked up only when the cursor enters it.  Every field is uniform across the wave.
  struct Cursor {
    int rg, ts, lo, hi, vrow, vstep;
    const unsigned char* kp;
    const unsigned char* vp;
  };
  auto range_start = [&](int rg) __attribute__((always_inline)) {
    Cursor c;
    c.rg = rg;
    if (rg == 0) {  // checkpoint cache: keys [slot rows, Hkv, D], values [slot, Hkv, D, cache_rows]
      c.ts = ts00, c.lo = lo0, c.hi = hi0, c.vrow = 2 * cache_rows, c.vstep = BN * 2;
      c.kp = reinterpret_cast<const unsigned char*>(k_cache + int64_t(kvh) * D + (int64_t(c.ts) + roff0) * Hkv * D);
      c.vp = reinterpret_cast<const unsigned char*>(v_cache + (int64_t(ckpt) * Hkv + kvh) * D * cache_rows +
                                                    int64_t(c.ts) + int64_t(w * IPW * 16) * cache_rows);
    } else {  // workspace: rotated keys, tile-major values (ts + voff is a multiple of 32)
      int64_t roff = roff1, voff = voff1;
      c.lo = lo1, c.hi = hi1;
      if (rg >= 2) {
        const int k = rg - 2;
        roff = own_word(k, TO_ROFF), voff = own_word(k, TO_VOFF);
        c.lo = max(own_word(k, TO_LO), lo_w), c.hi = own_word(k, TO_HI);
      }
      c.ts = c.lo & ~(BN - 1);
      c.vrow = BN * 2, c.vstep = D * BN * 2;
      c.kp = reinterpret_cast<const unsigned char*>(k_rot + int64_t(kvh) * D + (int64_t(c.ts) + roff) * Hkv * D);
      c.vp = reinterpret_cast<const unsigned char*>(vt + vt_index(kvh, w * IPW * 16, int64_t(c.ts) + voff, D, VT));
    }
    return c;
  };
  // the next tile (called only while one is left: the ranges hold n_tiles tiles in all)
  auto advance = [&](Cursor& c) __attribute__((always_inline)) {
    c.ts += BN;
    c.kp += int64_t(BN) * Hkv * D * 2;
    c.vp += c.vstep;
    if (__builtin_expect(c.ts >= c.hi, 0)) c = range_start(c.rg == 0 ? (n1 > 0 ? 1 : 2) : c.rg + 1);
  };
  // Lane constants of the copies: wave w issues copy instructions I = w*IPW + ii; lane l of
  // instruction I fills 16-byte LDS slot 64 I + l.  Key slot -> row k_row = I * 64 / KCH + l / KCH and
  // swizzled chunk; the swizzle of a row depends on its bits 0-1 and 3-4 only, so instruction
  // ii + KP reads the same chunk 4 rows further down.  Value slot -> channel row 16 I + l / 4 and
  // chunk vc, the same chunk for every instruction.
  constexpr int KP = 4 * KCH / 64;
  int k_off0[KP];
#pragma unroll
  for (int ii = 0; ii < KP; ++ii) {
    const int slot = (w * IPW + ii) * 64 + l;
    const int krow = slot / KCH;
    k_off0[ii] = (krow * Hkv * D + (((slot % KCH) ^ ksw(krow)) * 8)) * 2;  // bytes from the tile's first key row
  }
  const int vc = (l & 3) ^ vsw(l >> 2);
  auto issue = [&](const Cursor& c, int buf) {
    const int ts = c.ts, lo = c.lo, hi = c.hi, vrow = c.vrow;
    const bool edge = ts < lo || ts + BN > hi;
    unsigned char* kl = lds + buf * TILE_BYTES;
    unsigned char* vl = lds + (2 + buf) * TILE_BYTES;
    int lv = l;
    asm volatile("" : "+v"(lv));  // recomputed per tile: registers are scarce in the key-tile loop
    // the fixed key offsets are kept as 32-bit values inside the loop (which keeps the copies in their
    // scalar-base form instead of 64-bit lane addresses)
#pragma unroll
    for (int ii = 0; ii < KP; ++ii) asm volatile("" : "+v"(k_off0[ii]));
    // both offsets are >= 0 (clamped rows and chunks stay inside the range): 32-bit unsigned offsets
    // from a scalar base
    if (!edge) {
      // Interior tile: every per-instruction term goes into the scalar base, so the lane offsets are the
      // fixed key offsets and one value offset per tile.
      const uint32_t vlane = __umul24(uint32_t(lv >> 2), uint32_t(vrow)) + uint32_t(16 * vc);
#pragma unroll
      for (int ii = 0; ii < IPW; ++ii) {
        const unsigned char* kb = c.kp + uint32_t((ii / KP) * 4 * Hkv * D * 2);
        const unsigned char* vb = c.vp + uint32_t(ii * 16 * vrow);
        async_copy16(kb + uint32_t(k_off0[ii % KP]), kl + (w * IPW + ii) * 1024);
        async_copy16(vb + vlane, vl + (w * IPW + ii) * 1024);
      }
      asm volatile("");  // keeps this path's last copy out of a tail shared with the edge path
      return;
    }
    const int voff0 = (lv >> 2) * vrow + 16 * vc;
#pragma unroll
    for (int ii = 0; ii < IPW; ++ii) {  // masked keys read a valid row / value chunk of the range
      int koff = k_off0[ii % KP] + (ii / KP) * 4 * Hkv * D * 2;
      int voff = voff0 + ii * 16 * vrow;
      const int p = ts + ((w * IPW + ii) * 64 + lv) / KCH;
      const int pc = p < lo ? lo : (p >= hi ? hi - 1 : p);
      koff += (pc - p) * Hkv * D * 2;
      const int p0 = ts + 8 * vc;
      const int lo8 = lo & ~7, hi8 = (hi - 1) & ~7;
      const int p0c = p0 < lo8 ? lo8 : (p0 > hi8 ? hi8 : p0);
      voff += (p0c - p0) * 2;
      async_copy16(c.kp + uint32_t(koff), kl + (w * IPW + ii) * 1024);
      async_copy16(c.vp + uint32_t(voff), vl + (w * IPW + ii) * 1024);
    }
  };
  Cursor cur = range_start(n0 > 0 ? 0 : (n1 > 0 ? 1 : 2));  // the first tile (unused when there is none)

  // ---- rotated, pre-scaled queries as MFMA B fragments (query = column) ----
  // The rotation table rows of the tile's 32 positions are the same for every head: they are copied
  // once per workgroup into the second key and value buffers (rows 0-15 and 16-31; step 0 refills
  // those with tile 1 only after the barrier that follows every wave's rotation), 16-byte chunk x of
  // row r at slot x ^ (r % 16) so that the column reads of the rotation are conflict-free.  Rows past
  // the tile's end copy its first row; their queries are zeroed.
  constexpr int RB = D * 4;                 // bytes per table row: (cos, sin) in fp32 for D / 2 pairs
  constexpr int TCH = RB / 16;              // 16-byte chunks per table row
  constexpr int TPW = BN * RB / 1024 / 4;   // copy instructions per wave
  static_assert(BN * RB == 2 * TILE_BYTES && TCH >= 16, "table rows fill the second K and V buffers");
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int I = w * TPW + i;  // uniform: copy instruction I fills image bytes [1024 I, 1024 I + 1024)
    const int slot_img = I * 64 + l;
    const int row = slot_img / TCH, slot = slot_img % TCH;
    const int pos = row_info(row).pos;
    const unsigned char* src =
        reinterpret_cast<const unsigned char*>(table) + int64_t(pos) * RB + ((slot ^ (row & 15)) << 4);
    async_copy16(src, lds + (I * 1024 < TILE_BYTES ? TILE_BYTES + I * 1024 : 3 * TILE_BYTES + I * 1024 - TILE_BYTES));
  }
  const float sl2 = 1.4426950408889634f * rsqrtf(float(D));
  u32x4v qf[2][NC];
  int qrow[2];  // tile row of this lane's query column in block qb (its rotation table row)
  {
    u32x4v qa[2][NC / 2], qb_[2][NC / 2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int col = 32 * w + qb * 16 + r16;
      const int r = col / ng, hc = kvh * G + hg0 + col % ng;
      qrow[qb] = qvalid[qb] ? r : 0;
      const int64_t rowbase = (int64_t(col_info(col).row) * Hq + hc) * D + 8 * g4;
#pragma unroll
      for (int c = 0; c < NC / 2; ++c) {
        qa[qb][c] = *reinterpret_cast<const u32x4v*>(q + rowbase + 32 * c);
        qb_[qb][c] = *reinterpret_cast<const u32x4v*>(q + rowbase + 32 * c + D / 2);
      }
    }
    if (n_tiles > 0) issue(cur, 0);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's table rows (and everything else) have landed
    __syncthreads();                // ... and every wave's
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int rt = qrow[qb];  // table row (0 for columns past the tile)
      const bool qv = qvalid[qb];
      const unsigned char* trow = lds + (rt < 16 ? TILE_BYTES : 3 * TILE_BYTES) + (rt & 15) * RB;
#pragma unroll
      for (int c = 0; c < NC / 2; ++c) {
        u32x4v lo, hi;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const uint32_t av = qa[qb][c][ww], bv = qb_[qb][c][ww];
          const float a0 = __uint_as_float(av << 16), a1 = __uint_as_float(av & 0xFFFF0000u);
          const float b0 = __uint_as_float(bv << 16), b1 = __uint_as_float(bv & 0xFFFF0000u);
          // (cos, sin) of pairs 8 g4 + 32 c + 2 ww and the next one: chunk 4 g4 + 16 c + ww of the row
          const float4 t4 = *reinterpret_cast<const float4*>(trow + (((4 * g4 + 16 * c + ww) ^ (rt & 15)) << 4));
          lo[ww] = pack_bf16x2((a0 * t4.x - b0 * t4.y) * sl2, (a1 * t4.z - b1 * t4.w) * sl2);
          hi[ww] = pack_bf16x2((b0 * t4.x + a0 * t4.y) * sl2, (b1 * t4.z + a1 * t4.w) * sl2);
        }
        qf[qb][c] = qv ? lo : u32x4v{0u, 0u, 0u, 0u};
        qf[qb][c + NC / 2] = qv ? hi : u32x4v{0u, 0u, 0u, 0u};
      }
    }
  }

  f32x4v acc[2][NDB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x4v{0.f, 0.f, 0.f, 0.f};
  // m_run starts far below any score instead of at -inf: the first visible key always moves it, its
  // correction factor is then exactly 0 (as it would be from -inf), and no select is needed for the
  // exponent offset.  l_run: this lane's share of the column's sum.
  float m_run[2] = {-1e30f, -1e30f}, l_run[2] = {0.f, 0.f};
  // LDS byte offsets of this lane's MFMA operand reads.  Key fragment (kb, c) (key row
  // 8 (r16 / 4) + 4 kb + r16 % 4, chunk 4 c + g4 swizzled) sits at kfrag[c % 4] + kb * 4 * KROW +
  // 256 (c / 4): the swizzle is the same for both kb and only permutes chunk groups of four, so four
  // base offsets and immediate offsets cover all of them.  The V^T fragment of 16-channel block db
  // (channel row r16, keys 8 g4 .. +7) sits at vfrag + db * 16 * VROW.
  const int krow0 = 8 * (r16 >> 2) + (r16 & 3);
  const int ks = ksw(krow0);
  // (bits 6-7 of these offsets hold c % 4 ^ (ks >> 2) and nothing carries into them, so one base
  // and an XOR give all four)
  const int kfrag0 = krow0 * KROW + ((g4 ^ (ks & 3)) << 4) + ((ks >> 2) << 6);
  const int vfrag = r16 * VROW + ((g4 ^ vsw(r16)) << 4);
  const unsigned lds_base = unsigned(uintptr_t((__attribute__((address_space(3))) void*)lds));

  // One key tile.  Copies of tile t + 1 go out right after the barrier that frees their buffer; the
  // operand reads run a few fragments ahead of the MFMAs that use them, and the value reads of the
  // tile are issued before the softmax, which hides their latency.
  auto step = [&](int t, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of tile t have landed
    __syncthreads();                // ... and every wave's; buffer BUF ^ 1 is free
    const int ts = cur.ts, lo = cur.lo, hi = cur.hi, rg = cur.rg;
    if (t + 1 < n_tiles) {
      advance(cur);
      issue(cur, BUF ^ 1);
    }
    if (!active_s) return;
    if (rg >= 2 && !((own_mask >> (rg - 2)) & 1)) return;  // another question's own rows: none of this wave's keys
    // lane addresses of the operand reads (the array is 1024-byte aligned, so the chunk XOR of bits
    // 6-7 commutes with adding its base); tile, buffer and block offsets are instruction immediates
    int kf = kfrag0;
    asm volatile("" : "+v"(kf));  // keep the four XORs inside the loop (registers are scarce here)
    const unsigned kadr = lds_base + unsigned(kf), vadr = lds_base + unsigned(vfrag);
    auto kread = [&](auto J) {
      constexpr int j = decltype(J)::value, kb = j / NC, c = j % NC;
      return lds_read16<BUF * TILE_BYTES + kb * 4 * KROW + 256 * (c >> 2)>(kadr ^ unsigned((c & 3) << 6));
    };
    auto vread = [&](auto DB) {
      constexpr int db = decltype(DB)::value;
      return lds_read16<(2 + BUF) * TILE_BYTES + db * 16 * VROW>(vadr);
    };

    // S^T = K Q^T over the 32 keys of the tile (already in log2 units)
    f32x4v s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb][0] = s[kb][1] = f32x4v{0.f, 0.f, 0.f, 0.f};
    constexpr int KD = 3;  // operand reads in flight
    u32x4v fa[KD];
    static_for<0, KD>([&](auto J) { fa[decltype(J)::value] = kread(J); });
    // A wave in its score products issues ahead of the other wave of its SIMD, which is then mostly in
    // its softmax: the two overlap MFMA and VALU work better (2-3% on long-context rounds, measured).
    __builtin_amdgcn_s_setprio(1);
    static_for<0, 2 * NC>([&](auto J) {
      constexpr int j = decltype(J)::value, kb = j / NC, c = j % NC;
      lds_wait<(KD - 1 < 2 * NC - 1 - j ? KD - 1 : 2 * NC - 1 - j)>(fa[j % KD]);
      s[kb][0] = mfma16x16x32(fa[j % KD], qf[0][c], s[kb][0]);
      s[kb][1] = mfma16x16x32(fa[j % KD], qf[1][c], s[kb][1]);
      if constexpr (j + KD < 2 * NC) fa[j % KD] = kread(std::integral_constant<int, j + KD>{});
    });
    __builtin_amdgcn_s_setprio(0);
    u32x4v fv[KD];
    static_for<0, KD>([&](auto J) { fv[decltype(J)::value] = vread(J); });

    // mask: key p is visible to query column q iff kmin(q) <= p <= kmax(q)
    const bool full = ts >= lo && ts + BN <= hi && ts + BN - 1 <= qpos_min &&
                      (window == 0 || qpos_max - ts < window) && (rg < 2 || n_own == 1);
    u32x4v pf[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (!full) {
        const int kmin = window > 0 ? max(lo, qpos[qb] - window + 1) : lo;
        // an own range is visible to its own question's columns only
        const int kmax = rg >= 2 && qown[qb] != rg - 2 ? -1 : min(hi - 1, qpos[qb]);
        const uint32_t span = uint32_t(kmax - kmin);
        const int pb = ts + 8 * g4 - kmin;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = kmax >= kmin && uint32_t(pb + kb * 4 + i) <= span;
            s[kb][qb][i] = ok ? s[kb][qb][i] : -INFINITY;
          }
      }
      // The running maximum of a column moves only when the column's maximum grows by more than 8 (log2
      // units), which is when one of its four lanes' maxima does: the lanes compare their own 8 keys, and
      // the column maximum is formed only in the (rare) tiles where some lane of the wave moves.
      const float mx = fmaxf(fmaxf(fmaxf(s[0][qb][0], s[0][qb][1]), fmaxf(s[0][qb][2], s[0][qb][3])),
                             fmaxf(fmaxf(s[1][qb][0], s[1][qb][1]), fmaxf(s[1][qb][2], s[1][qb][3])));
      if (__builtin_amdgcn_ballot_w64(mx > m_run[qb] + 8.f)) {
        const float mc = rows4_max(mx);
        const float m_new = mc > m_run[qb] + 8.f ? fmaxf(m_run[qb], mc) : m_run[qb];
        const float corr = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        l_run[qb] *= corr;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[qb][db] *= corr;
        m_run[qb] = m_new;
      }
      const float m_use = m_run[qb];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kb][qb][i] = __builtin_amdgcn_exp2f(s[kb][qb][i] - m_use);
      pf[qb] = u32x4v{pack_bf16x2(s[0][qb][0], s[0][qb][1]), pack_bf16x2(s[0][qb][2], s[0][qb][3]),
                      pack_bf16x2(s[1][qb][0], s[1][qb][1]), pack_bf16x2(s[1][qb][2], s[1][qb][3])};
      // The column's sum takes the bf16 weights the output products use (so the weights of a column
      // sum to one up to fp32 rounding), two per instruction: this lane's 8 keys; the four lanes of a
      // column are summed once, at the end.
#pragma unroll
      for (int i = 0; i < 4; ++i) l_run[qb] = add_bf16_pair(pf[qb][i], l_run[qb]);
    }
    // O^T += V^T P^T over the tile's 32 keys (lane k-slots 8 g4 .. +7 = keys 8 g4 .. +7)
    static_for<0, NDB>([&](auto DB) {
      constexpr int db = decltype(DB)::value;
      lds_wait<(KD - 1 < NDB - 1 - db ? KD - 1 : NDB - 1 - db)>(fv[db % KD]);
      acc[0][db] = mfma16x16x32(fv[db % KD], pf[0], acc[0][db]);
      acc[1][db] = mfma16x16x32(fv[db % KD], pf[1], acc[1][db]);
      if constexpr (db + KD < NDB) fv[db % KD] = vread(std::integral_constant<int, db + KD>{});
    });
  };
  // unrolled by two so that each buffer's LDS offsets are immediates
  int t = 0;
  for (; t + 1 < n_tiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    step(t + 1, std::integral_constant<int, 1>{});
  }
  if (t < n_tiles) step(t, std::integral_constant<int, 0>{});

  // Output: each wave stages its 32 columns x D row-major in its quarter of the LDS (16-byte chunk c of
  // column k at slot c ^ (k % 16): conflict-free for both the 8-byte fragment writes and the 16-byte
  // reads), then stores whole head rows, 16 bytes per lane.  The accumulator layout would otherwise give
  // 8-byte pieces of sixteen rows per store.
  __syncthreads();  // every wave is done with the key and value tiles
  if (!active) return;
  constexpr int CPR = D / 8;  // 16-byte chunks per output row
  unsigned char* ow = lds + w * TILE_BYTES;  // BN == 32 rows of D: one wave's output tile
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qb * 16 + r16;  // staging row: the column's index in the wave
    const float l_col = rows4_sum(l_run[qb]);
    const float inv = col_info(32 * w + row).valid ? 1.f / l_col : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const f32x4v a = acc[qb][db];
      const int chunk = 2 * db + (g4 >> 1);
      *reinterpret_cast<u32x2v*>(ow + row * (D * 2) + ((chunk ^ (row & 15)) << 4) + ((g4 & 1) << 3)) =
          u32x2v{pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv)};
    }
  }
  constexpr int RPI = 64 / CPR;  // rows per 16-byte-per-lane read (a wave's LDS accesses run in order)
  const int c16 = l % CPR;
  if (ng == 4) {  // four heads: the wave's 32 columns are the 8 rows of unit w
    const int urow = unit_desc[4 * w + TU_ROW0], unr = unit_desc[4 * w + TU_NROWS];
#pragma unroll
    for (int k = 0; k < BN / RPI; ++k) {
      const int row = k * RPI + l / CPR;  // staging row = column 32 w + row: row row / 4 of unit w, head row % 4
      const u32x4v v = *reinterpret_cast<const u32x4v*>(ow + row * (D * 2) + ((c16 ^ (row & 15)) << 4));
      if (row / 4 < unr)
        *reinterpret_cast<u32x4v*>(o + (int64_t(urow + row / 4) * Hq + kvh * G + hg0 + row % 4) * D + c16 * 8) = v;
    }
  } else {
#pragma unroll
    for (int k = 0; k < BN / RPI; ++k) {
      const int row = k * RPI + l / CPR;  // staging row = column 32 w + row
      const u32x4v v = *reinterpret_cast<const u32x4v*>(ow + row * (D * 2) + ((c16 ^ (row & 15)) << 4));
      const int col = 32 * w + row, hc = kvh * G + hg0 + col % ng;
      const ColInfo ci = col_info(col);
      if (ci.valid) *reinterpret_cast<u32x4v*>(o + (int64_t(ci.row) * Hq + hc) * D + c16 * 8) = v;
    }
  }
}

bool attn_uses_mfma(const flide_attn_params& p) { return p.dtype == FLIDE_BF16 && (p.d == 256 || p.d == 128); }

int64_t attn_workspace_bytes(const flide_caps& c, const flide_attn_params& p) {
  const int64_t elem = p.dtype == FLIDE_BF16 ? 2 : 4;
  int64_t bytes = int64_t(c.T_cap) * p.Hkv * p.d * elem;  // rotated keys
  if (attn_uses_mfma(p)) {
    flide_meta_layout L;
    compute_layout(c, L);
    bytes += int64_t(p.Hkv) * p.d * vt_cols(c.T_cap, L.seg_cap) * elem;  // transposed values
  }
  return bytes;
}

int launch_attn_prepare(const MetaView& mv, const flide_attn_params& p, const RopeArgs& rope, const void* k,
                        const void* v, void* workspace, void* stream) {
  if (attn_uses_mfma(p)) {
    bf16_t* k_rot = (bf16_t*)workspace;
    bf16_t* vt = k_rot + int64_t(mv.T_cap) * p.Hkv * p.d;
    // row blocks rounded up to a multiple of kXcdClasses (see the id layout in kv_prep_kernel)
    dim3 pg(int((((mv.T_cap + 63) / 64 + kXcdClasses - 1) / kXcdClasses) * kXcdClasses) * p.Hkv);
    if (p.d == 256)
      hipLaunchKernelGGL(kv_prep_kernel<256>, pg, dim3(256), 0, (hipStream_t)stream, mv, (const bf16_t*)k,
                         (const bf16_t*)v, k_rot, vt, rope.table, rope.max_pos, p.Hkv);
    else
      hipLaunchKernelGGL(kv_prep_kernel<128>, pg, dim3(256), 0, (hipStream_t)stream, mv, (const bf16_t*)k,
                         (const bf16_t*)v, k_rot, vt, rope.table, rope.max_pos, p.Hkv);
    return int(hipGetLastError());
  }
  return launch_rope_k(mv, p, rope, k, workspace, stream);
}

// Interior checkpoint K/V: for every request that creates a checkpoint at save_m, the rotated keys and
// the values of positions 0..save_m-1 go to K/V cache slot save_slot, in the cache layouts (keys
// [slot][position][kv head][d], values [slot][kv head][d][position]).  Positions below the resume
// point m come from the cache slot the request resumed from, the others from this round's prepared
// workspace (rotated key rows; values transposed on the MFMA path, plain rows otherwise), so nothing is
// recomputed.  One workgroup per (request, kv head, 64 positions); the write slot differs from every
// slot read in the round (checked by the planner), and a slot or position outside the cache sets the
// device error word.
template <typename T, bool TRANSPOSED_V>
__global__ void __launch_bounds__(256) attn_save_kv_kernel(MetaView mv, const T* __restrict__ k_rot,
                                                           const T* __restrict__ vsrc, T* __restrict__ k_cache,
                                                           T* __restrict__ v_cache, int Hkv, int D, int cache_rows,
                                                           int cache_slots, int64_t VT) {
  const int j = blockIdx.x, g = blockIdx.y, p0 = blockIdx.z * 64;
  if (j >= mv.hdr[H_R]) return;
  const int slot = mv.req_save_slot[j];
  if (slot < 0) return;
  const int sm = mv.req_save_m[j], m = mv.req_m[j], ck = mv.req_ckpt[j];
  if (slot >= cache_slots || sm > cache_rows || (m > 0 && (ck < 0 || ck >= cache_slots))) {
    if (blockIdx.z == 0 && g == 0 && threadIdx.x == 0) flag_error(mv.dev_error, E_CACHE);
    return;
  }
  if (p0 >= sm) return;
  const int np = min(64, sm - p0);
  const int64_t row0 = mv.req_trunk_row0[j];
  const int64_t vcol0 = mv.seg_vcol0[j];  // trunk segment j: value column = vcol0 + position
  constexpr int EPC = 16 / int(sizeof(T));  // elements per 16-byte piece
  auto key_src = [&](int t) {
    return t < m ? k_cache + ((int64_t(ck) * cache_rows + t) * Hkv + g) * D : k_rot + ((row0 + t - m) * Hkv + g) * D;
  };
  if (D % EPC == 0) {  // keys: a row per position, d fastest, in 16-byte pieces
    const int cpr = D / EPC;
    for (int c = threadIdx.x; c < np * cpr; c += 256) {
      const int t = p0 + c / cpr, e0 = (c % cpr) * EPC;
      *reinterpret_cast<u32x4v*>(k_cache + ((int64_t(slot) * cache_rows + t) * Hkv + g) * D + e0) =
          *reinterpret_cast<const u32x4v*>(key_src(t) + e0);
    }
  } else {
    for (int idx = threadIdx.x; idx < np * D; idx += 256) {
      const int t = p0 + idx / D, dd = idx % D;
      k_cache[((int64_t(slot) * cache_rows + t) * Hkv + g) * D + dd] = key_src(t)[dd];
    }
  }
  auto value_at = [&](int dd, int t) {
    if (t < m) return v_cache[((int64_t(ck) * Hkv + g) * D + dd) * cache_rows + t];
    if (TRANSPOSED_V) return vsrc[vt_index(g, dd, vcol0 + t, D, VT)];
    return vsrc[((row0 + t - m) * Hkv + g) * D + dd];
  };
  // values: a row per channel, position fastest; a whole 16-byte piece of positions on one side of m is
  // one copy when both sides are transposed rows (piece starts are multiples of 8 positions: 16-byte
  // aligned in the cache and, with segment columns congruent to positions modulo 32, inside one column
  // block of the workspace), else element by element
  const int cpc = (np + EPC - 1) / EPC;
  for (int c = threadIdx.x; c < D * cpc; c += 256) {
    const int dd = c / cpc, t0 = p0 + (c % cpc) * EPC, n = min(EPC, p0 + np - t0);
    T* dst = v_cache + ((int64_t(slot) * Hkv + g) * D + dd) * cache_rows + t0;
    if (TRANSPOSED_V && n == EPC && (t0 + EPC <= m || t0 >= m)) {
      const T* src = t0 < m ? v_cache + ((int64_t(ck) * Hkv + g) * D + dd) * cache_rows + t0
                            : vsrc + vt_index(g, dd, vcol0 + t0, D, VT);
      *reinterpret_cast<u32x4v*>(dst) = *reinterpret_cast<const u32x4v*>(src);
    } else {
      for (int e = 0; e < n; ++e) dst[e] = value_at(dd, t0 + e);
    }
  }
}

int launch_attn_save_kv(const MetaView& mv, const flide_attn_params& p, const void* v, const void* workspace,
                        void* k_cache, void* v_cache, void* stream) {
  const dim3 grid(mv.R_cap, p.Hkv, (p.cache_rows + 63) / 64);
  hipStream_t st = (hipStream_t)stream;
  const int64_t krot_elems = int64_t(mv.T_cap) * p.Hkv * p.d;
  if (attn_uses_mfma(p)) {
    const bf16_t* k_rot = (const bf16_t*)workspace;
    hipLaunchKernelGGL((attn_save_kv_kernel<bf16_t, true>), grid, dim3(256), 0, st, mv, k_rot, k_rot + krot_elems,
                       (bf16_t*)k_cache, (bf16_t*)v_cache, p.Hkv, p.d, p.cache_rows, p.cache_slots,
                       vt_cols(mv.T_cap, mv.seg_cap));
  } else if (p.dtype == FLIDE_BF16) {
    hipLaunchKernelGGL((attn_save_kv_kernel<bf16_t, false>), grid, dim3(256), 0, st, mv, (const bf16_t*)workspace,
                       (const bf16_t*)v, (bf16_t*)k_cache, (bf16_t*)v_cache, p.Hkv, p.d, p.cache_rows,
                       p.cache_slots, int64_t(0));
  } else {
    hipLaunchKernelGGL((attn_save_kv_kernel<float, false>), grid, dim3(256), 0, st, mv, (const float*)workspace,
                       (const float*)v, (float*)k_cache, (float*)v_cache, p.Hkv, p.d, p.cache_rows, p.cache_slots,
                       int64_t(0));
  }
  return int(hipGetLastError());
}

int launch_attn_core(const MetaView& mv, const flide_attn_params& p, const RopeArgs& rope, const void* q,
                     const void* v, const void* k_cache, const void* v_cache, void* o, const void* workspace,
                     void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int W = p.window;
  if (attn_uses_mfma(p)) {
    const bf16_t* k_rot = (const bf16_t*)workspace;
    const bf16_t* vt = k_rot + int64_t(mv.T_cap) * p.Hkv * p.d;
    const int G = p.Hq / p.Hkv;
    dim3 grid(mv.tile_cap * p.Hkv * ((G + 3) / 4));  // tile_cap is a multiple of kXcdClasses
    auto kernel = p.d == 256 ? (G % 4 == 0 ? attn_mfma_kernel<256, true> : attn_mfma_kernel<256, false>)
                             : (G % 4 == 0 ? attn_mfma_kernel<128, true> : attn_mfma_kernel<128, false>);
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, st, mv, (const bf16_t*)q, k_rot, vt, (const bf16_t*)k_cache,
                       (const bf16_t*)v_cache, (bf16_t*)o, rope.table, rope.max_pos, p.Hq, p.Hkv, W, p.cache_rows,
                       p.cache_slots);
    return int(hipGetLastError());
  }
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
