// Row-wise layers of a multi-layer hybrid stack: RMSNorm, linear layers (x W^T, optionally plus a
// residual), SwiGLU and the GDN gates.
//
// Every layer other than the token mixers acts on each row alone ("Flide: Accelerating Decision
// Inference with Exact State Forking" §方法步骤详情, second step), so on the flat stream they run over its
// rows unchanged, and Proposition 3.1 carries over layer by layer.  After the last token mixer only the
// question-final rows are needed (§方法步骤详情, fourth step; Korean summary §어떻게 쓰나, selective
// readout): every kernel here takes a row set, all stream rows [0, T) or the question-final rows
// qfin_row[0 .. n_qst), read from the metadata, so a captured graph serves every round of its bucket.
#include "device_common.hpp"

namespace flide {

namespace {

// Row r of work index i, or -1 past the row set.
__device__ __forceinline__ int row_of(const MetaView& mv, int rows_mode, int i) {
  if (rows_mode == 0) return i < mv.hdr[H_T] ? i : -1;
  return i < mv.hdr[H_NQST] ? mv.qfin_row[i] : -1;
}

__device__ __forceinline__ float silu_f(float x) { return x / (1.f + __expf(-x)); }

// One wave per row: y = x / sqrt(mean(x^2) + eps) * g, accumulated in fp32.
template <typename T>
__global__ void __launch_bounds__(256) rmsnorm_kernel(MetaView mv, int rows_mode, const T* __restrict__ x,
                                                      const float* __restrict__ g, int D, float eps,
                                                      T* __restrict__ y) {
  const int r = row_of(mv, rows_mode, blockIdx.x * 4 + (threadIdx.x >> 6));
  if (r < 0) return;
  const int l = threadIdx.x & 63;
  const T* xr = x + int64_t(r) * D;
  float ss = 0.f;
  for (int e = l; e < D; e += 64) {
    const float v = load_f32(xr, e);
    ss += v * v;
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / float(D) + eps);
  T* yr = y + int64_t(r) * D;
  for (int e = l; e < D; e += 64) store_f32(yr, e, load_f32(xr, e) * inv * g[e]);
}

// out[r, f] = silu(gu[r, f]) * gu[r, F + f]
template <typename T>
__global__ void __launch_bounds__(256) swiglu_kernel(MetaView mv, int rows_mode, const T* __restrict__ gu, int F,
                                                     T* __restrict__ out) {
  const int r = row_of(mv, rows_mode, blockIdx.y);
  if (r < 0) return;
  for (int f = blockIdx.x * blockDim.x + threadIdx.x; f < F; f += gridDim.x * blockDim.x) {
    const float a = load_f32(gu, int64_t(r) * 2 * F + f), b = load_f32(gu, int64_t(r) * 2 * F + F + f);
    store_f32(out, int64_t(r) * F + f, silu_f(a) * b);
  }
}

// alpha = sigmoid(z[:, h] + bias[h]), eta = sigmoid(z[:, H + h] + bias[H + h]) over all stream rows
template <typename T>
__global__ void __launch_bounds__(256) gates_kernel(MetaView mv, const T* __restrict__ z,
                                                    const float* __restrict__ bias, int H, float* __restrict__ alpha,
                                                    float* __restrict__ eta) {
  const int T_rows = mv.hdr[H_T];
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < int64_t(T_rows) * H;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = i / H;
    const int h = int(i - r * H);
    const float a = load_f32(z, r * 2 * H + h) + bias[h];
    const float e = load_f32(z, r * 2 * H + H + h) + bias[H + h];
    alpha[i] = 1.f / (1.f + __expf(-a));
    eta[i] = 1.f / (1.f + __expf(-e));
  }
}

// ---- linear layers ----
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// C[r, n] = sum_k A[r, k] W[n, k] (+ R[r, n]), bf16 operands, fp32 accumulation on MFMA.
// Workgroup: 64 rows x 128 columns, 4 waves; wave w owns columns [32 w, 32 w + 32) of the tile, i.e.
// 4 x 2 blocks of 16 x 16.  K advances 32 at a time: the next step's A and W pieces (one and two 16-byte
// loads per thread) are loaded into registers while the MFMAs of the current step run on LDS.  Rows of
// A and C come from the row set; W rows past N and rows past the set read as zero and are not stored.
// K is a multiple of 32.  R may alias C (each element is read, then written, by the same thread).
constexpr int GM = 64, GN = 128, GK = 32;
constexpr int GLD = GK + 8;  // LDS row stride in bf16 (16 bytes of padding spread the fragment reads over the banks)

__global__ void __launch_bounds__(256) linear_mfma_kernel(MetaView mv, int rows_mode, const bf16_t* __restrict__ a,
                                                          int64_t lda, const bf16_t* __restrict__ w, int N, int K,
                                                          const bf16_t* R, bf16_t* C, int64_t ldc) {
  __shared__ __attribute__((aligned(16))) bf16_t As[GM * GLD];
  __shared__ __attribute__((aligned(16))) bf16_t Ws[GN * GLD];
  const int tid = threadIdx.x, l = tid & 63, wv = tid >> 6, r16 = l & 15, g4 = l >> 4;
  const int i0 = blockIdx.y * GM, n0 = blockIdx.x * GN;
  // this thread's pieces: A row ar (chunk ac), W rows wn0 and wn0 + 64 (chunk ac)
  const int ar = tid >> 2, ac = (tid & 3) * 8;
  const int arow = row_of(mv, rows_mode, i0 + ar);
  const int wn0 = n0 + ar, wn1 = n0 + ar + 64;
  const bf16_t* ap = arow >= 0 ? a + int64_t(arow) * lda + ac : nullptr;
  const bf16_t* wp0 = wn0 < N ? w + int64_t(wn0) * K + ac : nullptr;
  const bf16_t* wp1 = wn1 < N ? w + int64_t(wn1) * K + ac : nullptr;
  const u32x4v zero = {0u, 0u, 0u, 0u};
  u32x4v ra = ap ? *reinterpret_cast<const u32x4v*>(ap) : zero;
  u32x4v rw0 = wp0 ? *reinterpret_cast<const u32x4v*>(wp0) : zero;
  u32x4v rw1 = wp1 ? *reinterpret_cast<const u32x4v*>(wp1) : zero;
  f32x4v acc[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) acc[rb][0] = acc[rb][1] = f32x4v{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += GK) {
    __syncthreads();  // the previous step's fragment reads are done
    *reinterpret_cast<u32x4v*>(As + ar * GLD + ac) = ra;
    *reinterpret_cast<u32x4v*>(Ws + ar * GLD + ac) = rw0;
    *reinterpret_cast<u32x4v*>(Ws + (ar + 64) * GLD + ac) = rw1;
    __syncthreads();
    if (k0 + GK < K) {
      ra = ap ? *reinterpret_cast<const u32x4v*>(ap + k0 + GK) : zero;
      rw0 = wp0 ? *reinterpret_cast<const u32x4v*>(wp0 + k0 + GK) : zero;
      rw1 = wp1 ? *reinterpret_cast<const u32x4v*>(wp1 + k0 + GK) : zero;
    }
    // A fragment of row block rb: rows 16 rb + r16, k 8 g4 .. +7; W fragment of column block cb: columns
    // 32 wv + 16 cb + r16, the same k
    u32x4v fa[4], fw[2];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) fa[rb] = *reinterpret_cast<const u32x4v*>(As + (16 * rb + r16) * GLD + 8 * g4);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      fw[cb] = *reinterpret_cast<const u32x4v*>(Ws + (32 * wv + 16 * cb + r16) * GLD + 8 * g4);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, fa[rb]),
                                                              __builtin_bit_cast(bf16x8v, fw[cb]), acc[rb][cb], 0,
                                                              0, 0);
  }
  // explicit wait states before the VALU reads of the accumulators (the compiler's count was measured
  // short for a pack right after an MFMA elsewhere in this library)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2"
               : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]), "+v"(acc[2][0]),
                 "+v"(acc[2][1]), "+v"(acc[3][0]), "+v"(acc[3][1]));
  // lane holds C[16 rb + 4 g4 + i][32 wv + 16 cb + r16]
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row_of(mv, rows_mode, i0 + 16 * rb + 4 * g4 + i);
      if (r < 0) continue;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int n = n0 + 32 * wv + 16 * cb + r16;
        if (n >= N) continue;
        float v = acc[rb][cb][i];
        if (R) v += bf16_to_f32(R[int64_t(r) * ldc + n]);
        C[int64_t(r) * ldc + n] = f32_to_bf16(v);
      }
    }
}

// Larger form for K a multiple of 64: workgroup tile 128 rows x 128 columns, four waves of 64 x 64
// (4 x 4 blocks of 16 x 16), K advancing 64 at a time.  Both operand tiles are copied straight into LDS
// (16 bytes per lane) one K step ahead into the other of two buffers, with the 16-byte chunks of row r
// XOR-swizzled by (r / 2) % 8 so that the fragment reads (16 rows x 16 bytes per pass) are conflict-free;
// fragments are read with inline-asm ds_read_b128 and explicit lgkmcnt waits (the compiler would drain
// every LDS read behind the copies in flight).  Each output element accumulates the same 32-wide K chunks,
// in the same order, on the same MFMA as linear_mfma_kernel: the two forms give identical bits.
constexpr int TM = 128, TN = 128, TK = 64;
constexpr int TROW = TK * 2;        // bytes per tile row
constexpr int TBYTES = TM * TROW;   // bytes per operand tile (16 KB)

__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(src),
                                   (__attribute__((address_space(3))) void*)(lds_dst), 16, 0, 0);
}
template <int OFF>
__device__ __forceinline__ u32x4v ds_read16(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset field");
  u32x4v r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
// returns once at most N of this wave's LDS reads are outstanding, ordered before any use of the eight tied
// fragments
template <int N>
__device__ __forceinline__ void lgkm_wait8(u32x4v (&f)[8]) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5]), "+v"(f[6]), "+v"(f[7])
               : "i"(N));
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
linear_tile_kernel(MetaView mv, int rows_mode, const bf16_t* __restrict__ a, int64_t lda,
                   const bf16_t* __restrict__ w, int N, int K, const bf16_t* R, bf16_t* C, int64_t ldc) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * TBYTES];  // A0 W0 A1 W1
  const int tid = threadIdx.x, l = tid & 63, r16 = l & 15, g4 = l >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), wm = wv >> 1, wn = wv & 1;
  const int i0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  const int n_set = rows_mode == 0 ? mv.hdr[H_T] : mv.hdr[H_NQST];
  if (i0 >= n_set) return;  // the whole tile is past the row set
  // copies: instruction I = 4 wv + ii of an operand fills 16-byte slots 64 I + l, i.e. tile row 8 I + l / 8,
  // physical chunk l % 8 = logical chunk (l % 8) ^ ((row / 2) % 8).  Rows past the set or past N read a
  // valid row (their results are not stored).
  const bf16_t* asrc[4];
  const bf16_t* wsrc[4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int row = 8 * (4 * wv + ii) + (l >> 3);
    const int c = (l & 7) ^ ((row >> 1) & 7);
    int ar = row_of(mv, rows_mode, i0 + row);
    if (ar < 0) ar = row_of(mv, rows_mode, i0);
    const int wr = min(n0 + row, N - 1);
    asrc[ii] = a + int64_t(ar) * lda + 8 * c;
    wsrc[ii] = w + int64_t(wr) * K + 8 * c;
  }
  auto issue = [&](int k0, int stage) {
    unsigned char* at = lds + stage * 2 * TBYTES;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      copy16_to_lds(asrc[ii] + k0, at + (4 * wv + ii) * 1024);
      copy16_to_lds(wsrc[ii] + k0, at + TBYTES + (4 * wv + ii) * 1024);
    }
  };
  // fragment of row block b (rows 64 wm + 16 b + r16 of A, or 64 wn + 16 b + r16 of W), K half kk: logical
  // chunk 4 kk + g4 of the row; the swizzle of those rows is (r16 / 2) % 8
  const int swz = (r16 >> 1) & 7;
  const unsigned lds_base = unsigned(uintptr_t((__attribute__((address_space(3))) void*)lds));
  const unsigned abase = lds_base + unsigned((64 * wm + r16) * TROW);
  const unsigned wbase = lds_base + TBYTES + unsigned((64 * wn + r16) * TROW);
  const unsigned off0 = unsigned(((0 + g4) ^ swz) << 4), off1 = unsigned(((4 + g4) ^ swz) << 4);
  f32x4v acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4v{0.f, 0.f, 0.f, 0.f};
  auto step = [&](auto STAGE) {
    constexpr int SO = decltype(STAGE)::value * 2 * TBYTES;
    u32x4v f0[8], f1[8];  // K half 0 and 1: A blocks 0-3, then W blocks 0-3
    f0[0] = ds_read16<SO + 0 * 16 * TROW>(abase + off0);
    f0[1] = ds_read16<SO + 1 * 16 * TROW>(abase + off0);
    f0[2] = ds_read16<SO + 2 * 16 * TROW>(abase + off0);
    f0[3] = ds_read16<SO + 3 * 16 * TROW>(abase + off0);
    f0[4] = ds_read16<SO + 0 * 16 * TROW>(wbase + off0);
    f0[5] = ds_read16<SO + 1 * 16 * TROW>(wbase + off0);
    f0[6] = ds_read16<SO + 2 * 16 * TROW>(wbase + off0);
    f0[7] = ds_read16<SO + 3 * 16 * TROW>(wbase + off0);
    f1[0] = ds_read16<SO + 0 * 16 * TROW>(abase + off1);
    f1[1] = ds_read16<SO + 1 * 16 * TROW>(abase + off1);
    f1[2] = ds_read16<SO + 2 * 16 * TROW>(abase + off1);
    f1[3] = ds_read16<SO + 3 * 16 * TROW>(abase + off1);
    f1[4] = ds_read16<SO + 0 * 16 * TROW>(wbase + off1);
    f1[5] = ds_read16<SO + 1 * 16 * TROW>(wbase + off1);
    f1[6] = ds_read16<SO + 2 * 16 * TROW>(wbase + off1);
    f1[7] = ds_read16<SO + 3 * 16 * TROW>(wbase + off1);
    lgkm_wait8<8>(f0);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, f0[rb]),
                                                              __builtin_bit_cast(bf16x8v, f0[4 + cb]), acc[rb][cb], 0,
                                                              0, 0);
    lgkm_wait8<0>(f1);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, f1[rb]),
                                                              __builtin_bit_cast(bf16x8v, f1[4 + cb]), acc[rb][cb], 0,
                                                              0, 0);
  };
  const int nst = K / TK;
  issue(0, 0);
  for (int s0 = 0; s0 < nst; s0 += 2) {
    // stage s0 (buffer 0): its copies have landed everywhere; buffer 1 is free for stage s0 + 1
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (s0 + 1 < nst) issue((s0 + 1) * TK, 1);
    step(std::integral_constant<int, 0>{});
    if (s0 + 1 >= nst) break;
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (s0 + 2 < nst) issue((s0 + 2) * TK, 0);
    step(std::integral_constant<int, 1>{});
  }
  // explicit wait states before the VALU reads of the accumulators (see linear_mfma_kernel)
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2" : "+v"(acc[rb][0]), "+v"(acc[rb][1]), "+v"(acc[rb][2]), "+v"(acc[rb][3]));
  // lane holds C[64 wm + 16 rb + 4 g4 + i][64 wn + 16 cb + r16] of the tile
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row_of(mv, rows_mode, i0 + 64 * wm + 16 * rb + 4 * g4 + i);
      if (r < 0) continue;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int n = n0 + 64 * wn + 16 * cb + r16;
        if (n >= N) continue;
        float v = acc[rb][cb][i];
        if (R) v += bf16_to_f32(R[int64_t(r) * ldc + n]);
        C[int64_t(r) * ldc + n] = f32_to_bf16(v);
      }
    }
}

// fp32 linear layers: one output per thread, the K loop in order (fp32 mode is a correctness path).
__global__ void __launch_bounds__(256) linear_f32_kernel(MetaView mv, int rows_mode, const float* __restrict__ a,
                                                         int64_t lda, const float* __restrict__ w, int N, int K,
                                                         const float* R, float* C, int64_t ldc) {
  const int r = row_of(mv, rows_mode, blockIdx.y * 4 + (threadIdx.x >> 6));
  const int n = blockIdx.x * 64 + (threadIdx.x & 63);
  if (r < 0 || n >= N) return;
  const float* ar = a + int64_t(r) * lda;
  const float* wr = w + int64_t(n) * K;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc += ar[k] * wr[k];
  if (R) acc += R[int64_t(r) * ldc + n];
  C[int64_t(r) * ldc + n] = acc;
}

}  // namespace

int launch_rmsnorm(const MetaView& mv, int rows_mode, int dtype, int D, const void* x, const float* g, float eps,
                   void* y, void* stream) {
  const int n = rows_mode == 0 ? mv.T_cap : (mv.Q_cap > 0 ? mv.Q_cap : 1);
  const dim3 grid((n + 3) / 4);
  hipStream_t st = (hipStream_t)stream;
  if (dtype == FLIDE_BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, grid, dim3(256), 0, st, mv, rows_mode, (const bf16_t*)x, g, D, eps,
                       (bf16_t*)y);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, grid, dim3(256), 0, st, mv, rows_mode, (const float*)x, g, D, eps,
                       (float*)y);
  return int(hipGetLastError());
}

int launch_swiglu(const MetaView& mv, int rows_mode, int dtype, int F, const void* gu, void* out, void* stream) {
  const int n = rows_mode == 0 ? mv.T_cap : (mv.Q_cap > 0 ? mv.Q_cap : 1);
  const dim3 grid((F + 255) / 256, n);
  hipStream_t st = (hipStream_t)stream;
  if (dtype == FLIDE_BF16)
    hipLaunchKernelGGL(swiglu_kernel<bf16_t>, grid, dim3(256), 0, st, mv, rows_mode, (const bf16_t*)gu, F,
                       (bf16_t*)out);
  else
    hipLaunchKernelGGL(swiglu_kernel<float>, grid, dim3(256), 0, st, mv, rows_mode, (const float*)gu, F,
                       (float*)out);
  return int(hipGetLastError());
}

int launch_gates(const MetaView& mv, int dtype, int H, const void* z, const float* bias, float* alpha, float* eta,
                 void* stream) {
  int64_t work = int64_t(mv.T_cap) * H;
  int blocks = int((work + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == FLIDE_BF16)
    hipLaunchKernelGGL(gates_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, mv, (const bf16_t*)z, bias, H, alpha,
                       eta);
  else
    hipLaunchKernelGGL(gates_kernel<float>, dim3(blocks), dim3(256), 0, st, mv, (const float*)z, bias, H, alpha, eta);
  return int(hipGetLastError());
}

int launch_linear(const MetaView& mv, int rows_mode, int dtype, int N, int K, const void* a, int64_t lda,
                  const void* w, const void* resid, void* c, int64_t ldc, void* stream) {
  const int n = rows_mode == 0 ? mv.T_cap : (mv.Q_cap > 0 ? mv.Q_cap : 1);
  hipStream_t st = (hipStream_t)stream;
  if (dtype == FLIDE_BF16 && K % TK == 0) {
    const dim3 grid((N + TN - 1) / TN, (n + TM - 1) / TM);
    hipLaunchKernelGGL(linear_tile_kernel, grid, dim3(256), 0, st, mv, rows_mode, (const bf16_t*)a, lda,
                       (const bf16_t*)w, N, K, (const bf16_t*)resid, (bf16_t*)c, ldc);
  } else if (dtype == FLIDE_BF16) {
    const dim3 grid((N + GN - 1) / GN, (n + GM - 1) / GM);
    hipLaunchKernelGGL(linear_mfma_kernel, grid, dim3(256), 0, st, mv, rows_mode, (const bf16_t*)a, lda,
                       (const bf16_t*)w, N, K, (const bf16_t*)resid, (bf16_t*)c, ldc);
  } else {
    const dim3 grid((N + 63) / 64, (n + 3) / 4);
    hipLaunchKernelGGL(linear_f32_kernel, grid, dim3(256), 0, st, mv, rows_mode, (const float*)a, lda,
                       (const float*)w, N, K, (const float*)resid, (float*)c, ldc);
  }
  return int(hipGetLastError());
}

}  // namespace flide
