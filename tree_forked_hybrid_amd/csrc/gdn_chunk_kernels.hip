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
// Workgroup = (segment, head), 8 waves, one workgroup per CU (140 KB of LDS).  Wave w owns
// value channels [16w, 16w + 16) and the matching 16 rows of S, which stay in
// registers for the whole segment in the layout the next chunk's MFMA needs as
// its B operand.  Everything that depends on those channels (the values' conv,
// K S0^T, Q S0^T, the solve, O and the state update) is wave-local; only the
// channel-independent pieces (the normalised q/k tiles, A, Gamma (.) QK^T and
// the 16x16 diagonal inverses of I + A) are shared through LDS.  MFMA operands
// are fp16 (q, k are unit vectors; the other operands are O(1)); accumulation,
// the inverses and the state are fp32.
//
// Per chunk: (1) conv + L2 norm of q and k, one thread per (row quad, 8
// channels), the row norm summed over 16 lanes with DPP; values convolved by
// their owner wave straight into the solve's register layout; (2) Gram blocks
// A = KK^T and QK^T (the latter as hi*hi + hi*lo + lo*hi), K S0^T and Q S0^T,
// while one wave inverts the diagonal blocks of I + A in fp32; (3) A, P and
// K^T are written over the q/k lo tiles; (4) blocked forward substitution,
// outputs and the state update.
#include "device_common.hpp"

namespace flide {

int launch_gdn_plain(const MetaView& mv, const flide_gdn_params& p, int phase, const void* x, const float* conv_w,
                     const float* alpha, const float* eta, float* state_pool, void* conv_pool, int32_t n_slots,
                     void* o, void* stream);

namespace {

typedef _Float16 h4v __attribute__((ext_vector_type(4)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));

constexpr int CK = 64;   // chunk rows
constexpr int DK = 128;  // key size
constexpr int DV = 128;  // value size (8 waves x 16 channels)
constexpr int NT = 512;  // threads
constexpr int RAW_ROW = 3 * 128 * 2;  // bytes of one raw row of a head: q | k | v channels
// LDS stride of a raw row: 16 bytes of padding move each row 4 banks along, so the column reads of
// rows 4 apart (the value conv) fall in different banks
constexpr int RAW_STRIDE = RAW_ROW + 16;
constexpr int RAW_COPIES = ((CK + 3) * RAW_STRIDE + 1023) / 1024;  // 1 KB direct-to-LDS copies per chunk tile

__device__ __forceinline__ f4v mma16(h4v a, h4v b, f4v c) { return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0); }
__device__ __forceinline__ f4v mma32(h8v a, h8v b, f4v c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// Wait states between an MFMA and the first VALU read of its accumulator, issued explicitly.  With the
// wait states the compiler chose for a bf16 pack (v_cvt_pk_bf16_f32) eight slots after the last
// 16x16x16 MFMA of an output block, that pack read the accumulator before the MFMA had written it (the
// first two of the four rows a lane stores came out stale; measured on MI355X); 19 slots cover the
// longest MFMA of the kernel.
__device__ __forceinline__ void mfma_read_fence(f4v& v) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2" : "+v"(v)); }

__device__ __forceinline__ h4v to_h4(f4v v) { return h4v{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]}; }
__device__ __forceinline__ h8v cat8(h4v a, h4v b) { return h8v{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }
__device__ __forceinline__ h4v lds4(const _Float16* p) { return *reinterpret_cast<const h4v*>(p); }
__device__ __forceinline__ h8v lds8(const _Float16* p) { return *reinterpret_cast<const h8v*>(p); }

// Element offsets (in halves) inside the swizzled LDS tiles.  A [64][128] q/k
// tile keeps 16-byte chunk c of row t at chunk slot c ^ (t & 15); a [rows][64]
// tile (A, P, K^T) keeps chunk c of row r at c ^ ((r >> 1) & 7).  Both make the
// MFMA operand reads (16 rows x 16 or 8 bytes) bank-conflict free.
__device__ __forceinline__ int qk_off(int t, int c) { return t * DK + ((((c >> 3) ^ (t & 15))) << 3) + (c & 7); }
// The q/k tiles hold their key channels permuted within each block of 32: channel 32 b + 16 h + 4 g + i
// sits at column 32 b + 8 g + 4 h + i.  A 16-byte operand chunk 4 c + g4 then holds channels
// 32 c + 16 h + 4 g4 + i (h = 0, 1), exactly the k-slots of the state fragment built from the
// registers S[2 c], S[2 c + 1], so K S0^T and Q S0^T read each operand with one 16-byte access.  The
// Gram products contract both operands over the same columns and do not see the permutation.
__device__ __forceinline__ int dk_col(int x) {
  return (x & ~31) + (((x >> 2) & 3) << 3) + (((x >> 4) & 1) << 2) + (x & 3);
}
__device__ __forceinline__ int sq_off(int r, int c) { return r * CK + ((((c >> 3) ^ ((r >> 1) & 7))) << 3) + (c & 7); }

// Inclusive prefix sum over the 64 lanes on the VALU: shifts by 1, 2, 4 and 8 within each 16-lane row
// (lanes without a source add zero), then the last lane of row 0 / 2 is added to row 1 / 3 and the last
// lane of row 1 to rows 2 and 3.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v = dpp_add<0x111, 0xF>(v);  // row_shr:1
  v = dpp_add<0x112, 0xF>(v);  // row_shr:2
  v = dpp_add<0x114, 0xF>(v);  // row_shr:4
  v = dpp_add<0x118, 0xF>(v);  // row_shr:8
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  return dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
}

// sum over the 16 lanes of a DPP row (butterfly: quad swaps, half-row and row mirrors)
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));  // row_mirror
  return v;
}

// Targets of the direct-to-LDS copies, kept apart from the tiles so that the compiler can tell that
// no tile access touches them while copies are in flight.
struct ChunkIn {
  unsigned char raw[RAW_COPIES * 1024];  // raw rows c0 - 3 .. c0 + 63 of the head's q, k and v channels (bf16)
  float alpha[CK];                       // alpha and eta of the chunk's rows (0 past the segment)
  float eta[CK];
};

struct ChunkLds {
  _Float16 qh[CK * DK];  // normalised q, fp16 (hi part)
  _Float16 kh[CK * DK];  // normalised k, fp16 (hi part)
  _Float16 ql[CK * DK];  // q - hi (lo part)
  _Float16 kl[CK * DK];  // k - hi (lo part); after the Gram products: -A [t][s] then P [t][s]
  _Float16 kt[DK * CK];  // K^T [dk][t] (hi part), rows t permuted like the q/k columns (dk_col)
  _Float16 tinv[4][16][16];
  float cw[2][8][16][4];  // q/k conv taps [section][channel j][conv thread][tap] (tile writer's channel order), right-aligned
  alignas(16) float g[CK];    // g_t = sum of log alpha over the chunk's rows up to t
  alignas(16) float eta[CK];  // eta_t (0 past the chunk)
  alignas(16) float eg[CK];   // e^{g_t}
  alignas(16) float egn[CK];  // e^{g_n - g_t} (0 past the chunk)
  float egl;                  // e^{g_n}
};

// Workgroup barrier that orders LDS only: unlike __syncthreads() it does not wait for this wave's
// outstanding global loads, so the next chunk's direct-to-LDS copies stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.f + __expf(-v)); }

// lower-triangular 16-row block index -> (row block, column block)
template <int B>
struct Tri {
  static constexpr int ti = B >= 6 ? 3 : (B >= 3 ? 2 : (B >= 1 ? 1 : 0));
  static constexpr int si = B - ti * (ti + 1) / 2;
};

// Gram block B, transposed: the lane holds row t = 16 ti + r16, columns s = 16 si + 4 g4 + i.
// P blocks (Q K^T) use hi*hi + lo*hi + hi*lo: q.k of unit vectors can be far smaller than its
// fp16 rounding error; A blocks (K K^T) use hi*hi.
template <int B, bool IS_A>
__device__ __forceinline__ f4v gram_block(const ChunkLds& L, const int (&gq)[4]) {
  constexpr int rs = 16 * Tri<B>::si * DK, rt = 16 * Tri<B>::ti * DK;
  f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const h8v ks_ = lds8(L.kh + rs + gq[c]);
    if (IS_A) {
      acc = mma32(ks_, lds8(L.kh + rt + gq[c]), acc);
    } else {
      const h8v qt_ = lds8(L.qh + rt + gq[c]);
      acc = mma32(ks_, qt_, acc);
      acc = mma32(lds8(L.kl + rs + gq[c]), qt_, acc);
      acc = mma32(ks_, lds8(L.ql + rt + gq[c]), acc);
    }
  }
  return acc;
}

// decayed, masked Gram block -> fp16 rows of -A (s < t) or P (s <= t)
template <int B, bool IS_A>
__device__ __forceinline__ void gram_store(ChunkLds& L, f4v acc, int r16, int g4) {
  constexpr int ti = Tri<B>::ti, si = Tri<B>::si;
  const int t = 16 * ti + r16;
  const float gt = L.g[t], et = L.eta[t];
  h4v out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = 16 * si + 4 * g4 + i;
    const float dec = __expf(gt - L.g[s]);
    out[i] = IS_A ? (_Float16)(s < t ? -(et * dec * acc[i]) : 0.f) : (_Float16)(s <= t ? dec * acc[i] : 0.f);
  }
  // columns s permuted within blocks of 32 like the q/k columns (dk_col): s = 16 si + 4 g4 + i sits at
  // column 32 (si / 2) + 8 g4 + 4 (si % 2) + i; 16-byte chunks swizzled by row pair as in sq_off
  _Float16* base = IS_A ? L.kl : L.kl + CK * CK;
  *reinterpret_cast<h4v*>(base + 16 * ti * CK + r16 * CK + (((4 * (si >> 1) + g4) ^ ((r16 >> 1) & 7)) << 3) +
                          4 * (si & 1)) = out;
}

// One direct-to-LDS buffer load per lane of `BYTES` into the LDS address dst (lane i fills
// dst + BYTES * i); dst must be the same for every lane.
template <int BYTES>
__device__ __forceinline__ void lds_copy(__amdgpu_buffer_rsrc_t r, void* dst, int voff) {
  dma_to_lds<BYTES>(r, __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)dst),
                    voff);
}

// Direct-to-LDS copies for the chunk starting at segment row cc: raw rows cc - 3 .. cc + 63 of the
// head's q, k and v channels (rows outside the segment read as zero), and (wave 0) alpha, eta of rows
// cc .. cc + 63.  xs, as, es point at the segment's first raw row and its first alpha / eta entry of
// the head; head_b = byte offset of the head's q channels in a raw row, sect_b = bytes between the q, k
// and v sections, rowb = bytes per raw row, hstride = bytes between rows of alpha / eta.  Every buffer
// resource is based at the chunk (the raw one three rows before it, or at the segment start for the
// first chunk, whose rows -3 .. -1 then fall below the resource and read as zero), so no offset grows
// with the segment's length or the stream's capacity.
__device__ __forceinline__ void issue_chunk_loads(ChunkIn& I, const bf16_t* xs, const float* as, const float* es,
                                                  int len, int cc, int w, int l, int64_t rowb, int head_b, int sect_b,
                                                  int hstride) {
  const int nrow = min(len - cc, CK);  // >= 1
  if (w == 0) {
    const int64_t eoff = int64_t(cc) * hstride / 4;
    const int bytes = ((nrow - 1) * hstride / 4 + 1) * 4;
    const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc((void*)(as + eoff), 0, bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t er = __builtin_amdgcn_make_buffer_rsrc((void*)(es + eoff), 0, bytes, 0x00020000);
    lds_copy<4>(ar, I.alpha, l * hstride);
    lds_copy<4>(er, I.eta, l * hstride);
  }
  const int base_row = cc == 0 ? 0 : cc - 3;  // first raw row inside the resource
  const int nraw = min(len - base_row, CK + 3);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const unsigned char*>(xs) + int64_t(base_row) * rowb), 0, int(nraw * rowb), 0x00020000);
  const int rb32 = int(rowb);
  for (int cp = w; cp < RAW_COPIES; cp += NT / 64) {
    const int byte = cp * 1024 + 16 * l;
    const int row = byte / RAW_STRIDE, col = byte - row * RAW_STRIDE;
    const int chb = (col >> 8) * sect_b + head_b + (col & 255);
    // padding bytes and rows past the tile: zero fill (never read); rows before the segment have a
    // negative offset, which the hardware takes as a huge unsigned one: outside the resource, zero
    const int voff = row < CK + 3 && col < RAW_ROW ? (cc - 3 + row - base_row) * rb32 + chb : 0x7FFFFFF0;
    lds_copy<16>(xr, I.raw + cp * 1024, voff);
  }
}

// Row R of the substitution (the DPP broadcast lane must be a constant), then the next row.  T starts
// as the identity; row R becomes e_R - sum_{s<R} A[R][s] T[s][:].  A[R][s] is zero for s >= R (the
// block is strictly lower), so the products need no mask, and the identity entry of row R stays in
// place (every earlier row of column R is still zero).
template <int R>
struct InvRow {
  static __device__ __forceinline__ void run(const float (&av)[4], float (&tq)[4], int g4) {
    float part[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(av[i]), 0x150 + R, 0xF, 0xF, true));
      part[i] = a * tq[i];  // A[R][4 g4 + i] T[4 g4 + i][col]
    }
    const float tot = rows4_sum((part[0] + part[1]) + (part[2] + part[3]));
    if (g4 == (R >> 2)) tq[R & 3] -= tot;
    InvRow<R + 1>::run(av, tq, g4);
  }
};
template <>
struct InvRow<16> {
  static __device__ __forceinline__ void run(const float (&)[4], float (&)[4], int) {}
};

// Diagonal block B of A (fp32, from the hi tiles) and T_BB = (I + A_BB)^{-1} by forward
// substitution.  Lane (r16, g4) first holds A[r16][4 g4 + i]; for the substitution it owns column
// c = r16 and rows 4 g4 .. 4 g4 + 3 of T.  Row r of A reaches the lanes with a DPP row broadcast
// of lane r of every 16-lane row, each row of lanes sums its four products, and the four partial
// sums are combined across rows with lane swaps; nothing goes through LDS until T is stored.
template <int B>
__device__ __forceinline__ void diag_inverse(ChunkLds& L, const int (&gq)[4], int r16, int g4) {
  f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const h8v kb = lds8(L.kh + 16 * B * DK + gq[c]);
    acc = mma32(kb, kb, acc);
  }
  const int t = 16 * B + r16;
  const float gt = L.g[t], et = L.eta[t];
  float av[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = 16 * B + 4 * g4 + i;
    av[i] = s < t ? et * __expf(gt - L.g[s]) * acc[i] : 0.f;
  }
  const int col = r16;
  float tq[4];  // T[4 g4 + i][col], from the identity
#pragma unroll
  for (int i = 0; i < 4; ++i) tq[i] = 4 * g4 + i == col ? 1.f : 0.f;
  InvRow<0>::run(av, tq, g4);
#pragma unroll
  for (int i = 0; i < 4; ++i) L.tinv[B][4 * g4 + i][col] = (_Float16)tq[i];
}

}  // namespace

// PHASE 0: trunk segments (writes each request's state and conv window); PHASE 1: question segments.
// ACT 1: SiLU after the conv.
template <int PHASE, int ACT>
__global__ void __launch_bounds__(NT) gdn_chunk_kernel(MetaView mv, int H, int K,
                                                       const bf16_t* __restrict__ x, const float* __restrict__ conv_w,
                                                       const float* __restrict__ alpha,
                                                       const float* __restrict__ eta, float* __restrict__ state_pool,
                                                       bf16_t* __restrict__ conv_pool, int n_slots,
                                                       bf16_t* __restrict__ o, int det) {
  __shared__ ChunkLds L;
  __shared__ ChunkIn I;
  // workgroups are dispatched in linear order: rank = position in the longest-first work list
  const int lin = blockIdx.x + gridDim.x * blockIdx.y;
  const int item = lin / H, h = lin % H;
  const int R = mv.hdr[H_R];
  int seg;
  if (PHASE == 0) {
    if (item >= R) return;
    seg = mv.gdn_order[item];
  } else {
    if (item >= mv.hdr[H_NQST]) return;
    seg = mv.gdn_order[R + item];
  }
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g4 = l >> 4;
  const int64_t C = int64_t(H) * (2 * DK + DV);
  const int j = mv.seg_req[seg];
  const int row0 = mv.seg_row0[seg], len = mv.seg_len[seg];
  const int in_slot = mv.seg_state[seg];
  const int out_slot = PHASE == 0 ? mv.req_out[j] : -1;
  // an interior checkpoint of the trunk: its slot and the segment rows it covers (a chunk boundary)
  const int save_slot = PHASE == 0 ? mv.req_save_slot[j] : -1;
  const int save_rows = save_slot >= 0 ? mv.req_save_m[j] - mv.req_m[j] : -1;
  if (in_slot >= n_slots || out_slot >= n_slots || save_slot >= n_slots || (PHASE == 1 && in_slot < 0)) {
    if (tid == 0) flag_error(mv.dev_error, E_SLOT);
    return;
  }
  const bf16_t* hist = in_slot >= 0 ? conv_pool + int64_t(in_slot) * (K - 1) * C : nullptr;
  const int qch = h * DK, kch = H * DK + h * DK, vch = 2 * H * DK + h * DV;
  const int ncol = 16 * w + r16;  // this lane's value channel / state row

  // Raw inputs through buffer resources: the segment's rows [0, len) and the conv history window
  // (K - 1 rows before the segment).  A row outside either reads as zero (out-of-range buffer
  // loads return 0; a negative byte offset wraps past the end), which is the conv's zero padding.
  const int rowb = int(C) * 2;  // bytes per raw row
  const bf16_t* const xs = x + int64_t(row0) * C;
  const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(hist != nullptr ? hist : x), 0, hist != nullptr ? (K - 1) * rowb : 0, 0x00020000);
  const int hoff = (K - 1) * rowb;  // byte offset of segment row 0 in the history window's row numbering

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
  constexpr float kQkTapScale = ACT == 1 ? 1.4426950408889634f : 1.f;
  // q/k conv threads: waves 0-3 -> q, 4-7 -> k; row quad rq (rows 4 rq .. 4 rq + 3), channels 8 r16 .. 8 r16 + 7
  const int sec = w >> 2, rq = (w & 3) * 4 + g4, p8 = 32 * (r16 >> 2) + 4 * (r16 & 3);
  for (int it = tid; it < 2 * DK * 4; it += NT) {
    const int ci = it >> 2, tap = it & 3;
    const int sc = ci / DK, cc = ci % DK;
    const int tau = tap - (4 - K);
    // channel cc = 32 b + 16 h + 4 g + i is channel 4 h + i of conv thread 4 b + g (see the tile writer);
    // with SiLU the taps carry a factor log2(e) (the conv's output then feeds exp2 directly)
    L.cw[sc][4 * ((cc >> 4) & 1) + (cc & 3)][4 * (cc >> 5) + ((cc >> 2) & 3)][tap] =
        tau >= 0 ? kQkTapScale * conv_w[int64_t((sc ? kch : qch) + cc) * K + tau] : 0.f;
  }
  float vw[4];  // this lane's value-channel taps, right-aligned
#pragma unroll
  for (int tap = 0; tap < 4; ++tap) {
    const int tau = tap - (4 - K);
    vw[tap] = tau >= 0 ? conv_w[int64_t(vch + ncol) * K + tau] : 0.f;
  }
  // lane offsets (halves) into the swizzled tiles, for rows 16 x + r16 (add 16 x * row length):
  // q/k tile, 16-byte operand chunk 4 c + g4
  int gq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) gq[c] = r16 * DK + ((((4 * c + g4) ^ r16)) << 3);

  // The copies of the next chunk are issued once the current chunk's conv is done with the tile; the
  // first chunk's history rows are patched in at its top.
  const float* const as = alpha + int64_t(row0) * H + h;
  const float* const es = eta + int64_t(row0) * H + h;
  const int head_b = h * DK * 2, sect_b = H * DK * 2;
  const int rowo = H * DV * 2;  // bytes per output row
  if (len > 0) issue_chunk_loads(I, xs, as, es, len, 0, w, l, rowb, head_b, sect_b, H * 4);
  // rows -3 .. -1 of the first chunk: the conv history window (K - 1 rows; older rows stay zero), loaded
  // beside the first chunk's copies and patched into the tile once those have landed
  constexpr int HIST_THREADS = 3 * RAW_ROW / 16;
  u4v hist_v = {0u, 0u, 0u, 0u};
  if (hist != nullptr && tid < HIST_THREADS) {
    const int row = tid / (RAW_ROW / 16), col = (tid % (RAW_ROW / 16)) * 16;
    const int chb = (col >> 8) * sect_b + head_b + (col & 255);
    hist_v = __builtin_amdgcn_raw_buffer_load_b128(hr, (row - 3) * rowb + hoff + chb, 0, 0);
  }

  _Float16* const am = L.kl;           // -A [t][s] (strictly lower blocks), after the Gram products
  _Float16* const pm = L.kl + CK * CK;  // P [t][s] (lower blocks)

  // Chunk boundaries: every 64 rows from the segment's first row (det != 0: the arithmetic of a segment
  // depends on the segment alone), or at the multiples of 64 stream rows and at an interior checkpoint
  // (det == 0: the grid of a packed batch, under which a segment's bits depend on where it lands).
  for (int c0 = 0, n = 0; c0 < len; c0 += n) {
    n = min(CK, len - c0);
    if (!det) {
      n = min(n, CK - ((row0 + c0) & (CK - 1)));
      if (save_rows > c0) n = min(n, save_rows - c0);
    }
    // Lane indices recomputed per chunk from an opaque copy: the per-lane LDS addresses derived from
    // them below are cheap to rebuild, and keeping them out of the loop preheader keeps them out of
    // registers across the whole segment.
    int tid_v = tid;
    asm volatile("" : "+v"(tid_v));
    const int l = tid_v & 63, r16 = l & 15, g4 = l >> 4;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed
    lds_barrier();                  // ... and every wave's; the previous chunk is done with the LDS tiles
    if (c0 == 0 && hist != nullptr) {
      if (tid_v < HIST_THREADS) {
        const int row = tid_v / (RAW_ROW / 16), col = (tid_v % (RAW_ROW / 16)) * 16;
        *reinterpret_cast<u4v*>(I.raw + row * RAW_STRIDE + col) = hist_v;
      }
      lds_barrier();
    }
    uint32_t vraw[4][7];  // bf16 bits of this lane's value channel at tile rows 16 rb + 4 g4 + i
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 7; ++i)
        vraw[rb][i] = *reinterpret_cast<const unsigned short*>(I.raw + (16 * rb + 4 * g4 + i) * RAW_STRIDE + 512 + 2 * ncol);
    // this thread's q/k row window at tile rows 4 rq + i: channels 32 b + 4 g + (0..3) and 32 b + 16 + 4 g + (0..3)
    // for r16 = 4 b + g, the two halves of one 16-byte operand chunk of the permuted tiles (dk_col)
    u4v raw[7];
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      const unsigned char* rp = I.raw + (4 * rq + i) * RAW_STRIDE + sec * 256 + 2 * p8;
      const u2v a = *reinterpret_cast<const u2v*>(rp), b = *reinterpret_cast<const u2v*>(rp + 32);
      raw[i] = u4v{a[0], a[1], b[0], b[1]};
    }
    if (w == 0) {
      // g = inclusive prefix sum of log alpha over the chunk
      const int t = l;
      const float e = t < n ? I.eta[t] : 0.f;
      float gsum = t < n ? __logf(I.alpha[t]) : 0.f;
      gsum = wave_prefix_sum(gsum);
      const float gn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gsum), n - 1));
      L.g[t] = gsum;
      L.eta[t] = e;
      L.eg[t] = __expf(gsum);
      L.egn[t] = t < n ? __expf(gn - gsum) : 0.f;
      if (t == 0) L.egl = __expf(gn);
    }
    // ---- values of this lane's channel at rows 16 rb + 4 g4 + i (the solve's layout) ----
    // (computed at the end of each wave's share of the Gram stage, pinned there: left to the compiler
    // it lands after the K S0^T products)
    f4v vv[4];
    auto value_conv = [&]() {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          auto xv = [&](int k) { return __uint_as_float(vraw[rb][k] << 16); };
          float acc = vw[0] * xv(i) + vw[1] * xv(i + 1) + vw[2] * xv(i + 2) + vw[3] * xv(i + 3);
          if (ACT == 1) acc = silu(acc);
          vv[rb][i] = acc;
        }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) asm volatile("" : "+v"(vv[rb]));
    };
    // ---- conv + L2 norm of q and k -> fp16 hi/lo tiles ----
    {
      _Float16* th = sec ? L.kh : L.qh;
      _Float16* tl = sec ? L.kl : L.ql;
      float4 wt4[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) wt4[c] = *reinterpret_cast<const float4*>(L.cw[sec][c][r16]);
      h4v kcol[8];  // hi values of the thread's channels at its four rows
#pragma unroll
      for (int jr = 0; jr < 4; ++jr) {
        const int t = 4 * rq + jr;
        float y[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float4 wt = wt4[c];
          const int hw = c >> 1;
          auto xv = [&](int i) {
            const uint32_t wv = raw[i][hw];
            return (c & 1) ? __uint_as_float(wv & 0xFFFF0000u) : __uint_as_float(wv << 16);
          };
          float acc = wt.x * xv(jr) + wt.y * xv(jr + 1) + wt.z * xv(jr + 2) + wt.w * xv(jr + 3);
          // SiLU of u = acc / log2(e), times log2(e): acc sigmoid(u), with e^-u = 2^-acc
          if (ACT == 1) acc *= __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-acc));
          y[c] = acc;
        }
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) ss += y[c] * y[c];
        ss = row16_sum(ss);
        // the L2 norm is blind to the common factor log2(e) but for its epsilon, scaled to match
        const float inv = t < n ? rsqrtf(ss + 1e-6f * kQkTapScale * kQkTapScale) : 0.f;
        h8v hv, lv;
#pragma unroll
        for (int c = 0; c < 8; ++c) {  // hi and lo of y inv, each one fused multiply-add rounded to fp16
          const _Float16 hi = (_Float16)__builtin_fmaf(y[c], inv, 0.f);
          hv[c] = hi;
          lv[c] = (_Float16)__builtin_fmaf(y[c], inv, -(float)hi);
        }
        // the thread's 8 channels are exactly the permuted tile's chunk r16 (dk_col)
        const int wo = t * DK + ((r16 ^ (4 * g4 + jr)) << 3);
        *reinterpret_cast<h8v*>(th + wo) = hv;
        *reinterpret_cast<h8v*>(tl + wo) = lv;
#pragma unroll
        for (int c = 0; c < 8; ++c) kcol[c][jr] = hv[c];
      }
      if (sec == 1) {  // K^T: the k threads hold four consecutive rows of each of their 8 channels
        const int t0 = 4 * rq;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int dk = 32 * (r16 >> 2) + 4 * (r16 & 3) + 16 * (c >> 2) + (c & 3);
          *reinterpret_cast<h4v*>(L.kt + sq_off(dk, dk_col(t0))) = kcol[c];
        }
      }
    }
    lds_barrier();
    if (c0 + n < len) issue_chunk_loads(I, xs, as, es, len, c0 + n, w, l, rowb, head_b, sect_b, H * 4);
    // ---- Gram blocks, held in registers until every wave is done with the lo tiles.  Waves 4-7 take
    // two P blocks and one strictly lower A block each; waves 0-3 one remaining block and, one each,
    // the diagonal A blocks and their inverses: the substitution chain runs on the older wave of each
    // SIMD, which the hardware issues first ----
    f4v gres[3];
    switch (w ^ 4) {
      case 0: gres[0] = gram_block<0, false>(L, gq); gres[1] = gram_block<4, false>(L, gq);
              gres[2] = gram_block<1, true>(L, gq); value_conv(); break;
      case 1: gres[0] = gram_block<1, false>(L, gq); gres[1] = gram_block<5, false>(L, gq);
              gres[2] = gram_block<3, true>(L, gq); value_conv(); break;
      case 2: gres[0] = gram_block<2, false>(L, gq); gres[1] = gram_block<6, false>(L, gq);
              gres[2] = gram_block<6, true>(L, gq); value_conv(); break;
      case 3: gres[0] = gram_block<3, false>(L, gq); gres[1] = gram_block<7, false>(L, gq);
              gres[2] = gram_block<7, true>(L, gq); value_conv(); break;
      case 4: gres[0] = gram_block<8, false>(L, gq); diag_inverse<0>(L, gq, r16, g4); value_conv(); break;
      case 5: gres[0] = gram_block<9, false>(L, gq); diag_inverse<1>(L, gq, r16, g4); value_conv(); break;
      case 6: gres[0] = gram_block<4, true>(L, gq); diag_inverse<2>(L, gq, r16, g4); value_conv(); break;
      default: gres[0] = gram_block<8, true>(L, gq); diag_inverse<3>(L, gq, r16, g4); value_conv(); break;
    }
    // ---- K S0^T and Q S0^T for this wave's channels, and the solve's right-hand side ----
    h8v sf[4];  // S as the B operand (k-slots permuted to match the register layout)
#pragma unroll
    for (int c = 0; c < 4; ++c) sf[c] = cat8(to_h4(S[2 * c]), to_h4(S[2 * c + 1]));
    f4v qs[4], rhs[4];
    const bool zero_state = c0 == 0 && in_slot < 0;  // a fresh trunk's first chunk: both products vanish
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f4v ks = {0.f, 0.f, 0.f, 0.f};
      qs[rb] = f4v{0.f, 0.f, 0.f, 0.f};
      if (!zero_state) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          ks = mma32(lds8(L.kh + 16 * rb * DK + gq[c]), sf[c], ks);
          qs[rb] = mma32(lds8(L.qh + 16 * rb * DK + gq[c]), sf[c], qs[rb]);
        }
      }
      const f4v eg4 = *reinterpret_cast<const f4v*>(&L.eg[16 * rb + 4 * g4]);
      const f4v eta4 = *reinterpret_cast<const f4v*>(&L.eta[16 * rb + 4 * g4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) rhs[rb][i] = eta4[i] * (vv[rb][i] - eg4[i] * ks[i]);
    }
    lds_barrier();  // every wave is done with the lo tiles; the diagonal inverses are in LDS
    // ---- -A and P over the lo tiles ----
    switch (w ^ 4) {
      case 0: gram_store<0, false>(L, gres[0], r16, g4); gram_store<4, false>(L, gres[1], r16, g4);
              gram_store<1, true>(L, gres[2], r16, g4); break;
      case 1: gram_store<1, false>(L, gres[0], r16, g4); gram_store<5, false>(L, gres[1], r16, g4);
              gram_store<3, true>(L, gres[2], r16, g4); break;
      case 2: gram_store<2, false>(L, gres[0], r16, g4); gram_store<6, false>(L, gres[1], r16, g4);
              gram_store<6, true>(L, gres[2], r16, g4); break;
      case 3: gram_store<3, false>(L, gres[0], r16, g4); gram_store<7, false>(L, gres[1], r16, g4);
              gram_store<7, true>(L, gres[2], r16, g4); break;
      case 4: gram_store<8, false>(L, gres[0], r16, g4); break;
      case 5: gram_store<9, false>(L, gres[0], r16, g4); break;
      case 6: gram_store<4, true>(L, gres[0], r16, g4); break;
      default: gram_store<8, true>(L, gres[0], r16, g4); break;
    }
    // The state after a question's last chunk is not kept (only trunks emit a state), so the question
    // call skips the state update there.
    const bool keep_state = PHASE == 0 || c0 + n < len;
    lds_barrier();
    // ---- blocked forward substitution U = (I + A)^{-1} RHS ----
    h4v uh[4];
    f4v u[4];
    // Rows of -A and P hold their columns s permuted within blocks of 32 (gram_store), so two 16-column
    // blocks jb = 2 p, 2 p + 1 are one 16-byte operand chunk 4 p + g4 against cat8(uh[2 p], uh[2 p + 1]);
    // a lone block jb is the 8-byte half 4 (jb % 2) of chunk 4 (jb / 2) + g4.
    const int swz = (r16 >> 1) & 7;
    auto pair_off = [&](int p2) { return r16 * CK + (((4 * p2 + g4) ^ swz) << 3); };
    auto half_off = [&](int jb) { return r16 * CK + (((4 * (jb >> 1) + g4) ^ swz) << 3) + 4 * (jb & 1); };
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f4v acc = rhs[rb];
#pragma unroll
      for (int p2 = 0; 2 * p2 + 1 < rb; ++p2)
        acc = mma32(lds8(am + 16 * rb * CK + pair_off(p2)), cat8(uh[2 * p2], uh[2 * p2 + 1]), acc);
      if (rb & 1) acc = mma16(lds4(am + 16 * rb * CK + half_off(rb - 1)), uh[rb - 1], acc);
      if (rb > 0) mfma_read_fence(acc);
      u[rb] = mma16(lds4(&L.tinv[rb][r16][4 * g4]), to_h4(acc), f4v{0.f, 0.f, 0.f, 0.f});
      mfma_read_fence(u[rb]);
      uh[rb] = to_h4(u[rb]);
    }
    // ---- outputs O = e^g Q S0^T + P U ----
    // rows of this chunk only: stores past the segment fall outside the resource
    const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(o + (int64_t(row0) + c0) * H * DV), 0, n * rowo, 0x00020000);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f4v acc = *reinterpret_cast<const f4v*>(&L.eg[16 * rb + 4 * g4]) * qs[rb];
#pragma unroll
      for (int p2 = 0; 2 * p2 + 1 <= rb; ++p2)
        acc = mma32(lds8(pm + 16 * rb * CK + pair_off(p2)), cat8(uh[2 * p2], uh[2 * p2 + 1]), acc);
      if ((rb & 1) == 0) acc = mma16(lds4(pm + 16 * rb * CK + half_off(rb)), uh[rb], acc);
      mfma_read_fence(acc);
      const uint32_t p01 = pack_bf16x2(acc[0], acc[1]), p23 = pack_bf16x2(acc[2], acc[3]);
      const int ob = (16 * rb + 4 * g4) * rowo + (h * DV + ncol) * 2;  // row 16 rb + 4 g4 of this chunk
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)p01, orr, ob, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(p01 >> 16), orr, ob + rowo, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)p23, orr, ob + 2 * rowo, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(p23 >> 16), orr, ob + 3 * rowo, 0, 0);
    }
    // ---- state update S = e^{g_n} S + U^T diag(e^{g_n - g}) K ----
    if (!keep_state) continue;
    h4v ud[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const f4v egn4 = *reinterpret_cast<const f4v*>(&L.egn[16 * rb + 4 * g4]);
      // rows past the chunk contribute nothing: egn is 0 there, and u is exactly 0 (eta = 0 makes their
      // right-hand sides and their rows of A vanish)
      ud[rb] = to_h4(egn4 * u[rb]);
    }
    const float egl = L.egl;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      f4v acc = S[mb] * egl;
      // rows t of K^T are permuted within blocks of 32 (dk_col), so chunk 4 p + g4 of a K^T row holds
      // t = 32 p + 16 h + 4 g4 + i, the k-slots of cat8(ud[2 p], ud[2 p + 1])
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2)
        acc = mma32(lds8(L.kt + 16 * mb * CK + r16 * CK + (((4 * p2 + g4) ^ ((r16 >> 1) & 7)) << 3)),
                    cat8(ud[2 * p2], ud[2 * p2 + 1]), acc);
      S[mb] = acc;
    }
    if (PHASE == 0 && c0 + n == save_rows) {  // the checkpoint's state: S after this chunk's last row
      float* sdst = state_pool + ((int64_t(save_slot) * H + h) * DV + ncol) * DK;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) *reinterpret_cast<f4v*>(sdst + 16 * mb + 4 * g4) = S[mb];
    }
  }

  if (PHASE == 0) {
    float* dst = state_pool + ((int64_t(out_slot) * H + h) * DV + ncol) * DK;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) *reinterpret_cast<f4v*>(dst + 16 * mb + 4 * g4) = S[mb];
    // conv window: the K-1 raw inputs of (history ++ segment) before segment row `upto`, over the
    // head's q, k and v channels; for the trunk's end and for an interior checkpoint
    auto write_window = [&](int slot, int upto) {
      bf16_t* wdst = conv_pool + int64_t(slot) * (K - 1) * C;
      const int nch = 2 * DK + DV;
      for (int it = tid; it < (K - 1) * nch; it += NT) {
        const int wr = it / nch, ci = it - wr * nch;
        const int ch = ci < DK ? qch + ci : (ci < 2 * DK ? kch + ci - DK : vch + ci - 2 * DK);
        const int u = upto - (K - 1) + wr;
        bf16_t val = 0;
        if (u >= 0)
          val = x[int64_t(row0 + u) * C + ch];
        else if (hist != nullptr)
          val = hist[int64_t(K - 1 + u) * C + ch];
        wdst[int64_t(wr) * C + ch] = val;
      }
    };
    write_window(out_slot, len);
    if (save_slot >= 0) write_window(save_slot, save_rows);
  }
}

bool gdn_uses_chunk(const flide_gdn_params& p) { return p.dtype == FLIDE_BF16 && p.dk == DK && p.dv == DV; }

int launch_gdn(const MetaView& mv, const flide_gdn_params& p, int phase, const void* x, const float* conv_w,
               const float* alpha, const float* eta, float* state_pool, void* conv_pool, int32_t n_slots, void* o,
               void* stream) {
  // (buffer offsets of the chunk kernel are relative to each chunk: any capacity and segment length)
  if (!gdn_uses_chunk(p))
    return launch_gdn_plain(mv, p, phase, x, conv_w, alpha, eta, state_pool, conv_pool, n_slots, o, stream);
  dim3 grid(phase == 0 ? mv.R_cap : (mv.Q_cap > 0 ? mv.Q_cap : 1), p.H);
  auto kern = phase == 0 ? (p.act == 1 ? gdn_chunk_kernel<0, 1> : gdn_chunk_kernel<0, 0>)
                        : (p.act == 1 ? gdn_chunk_kernel<1, 1> : gdn_chunk_kernel<1, 0>);
  hipLaunchKernelGGL(kern, grid, dim3(NT), 0, (hipStream_t)stream, mv, p.H, p.conv_k,
                     (const bf16_t*)x, conv_w, alpha, eta, state_pool, (bf16_t*)conv_pool, n_slots, (bf16_t*)o,
                     p.deterministic != 0 ? 1 : 0);
  return int(hipGetLastError());
}

}  // namespace flide
