// C ABI: context, validation, kernel dispatch and graph buckets.
//
// Flat-graph execution (Korean summary §어떻게 쓰나; "Flide: Accelerating
// Decision Inference with Exact State Forking" §核心方法 and §方法步骤详情,
// third step): one HIP graph is captured per stream capacity; a round writes
// its metadata into the bucket's device buffer (one small host-to-device copy
// from pinned staging) and replays the graph.  Kernels size their work from
// the metadata, so the launch shapes depend only on the capacity.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "flide_internal.hpp"

using namespace flide;

namespace {

struct RopeTable {
  double theta;
  int d;
  int max_pos;
  float* dev;
};

struct Staging {
  int32_t* host[2] = {nullptr, nullptr};
  hipEvent_t done[2] = {nullptr, nullptr};
  int64_t words = 0;
  int next = 0;
};

// A captured bucket: the round in four graphs (parts), replayed in part order or split over streams:
// 0 metadata expansion, 1 the trunk GDN call, 2 attention and checkpoint K/V, 3 the question GDN call and
// the readout.  Parts 1 and 2 read only the expanded metadata and the round's inputs, so a caller may run
// them side by side; part 3 needs part 1 (flide_graph_replay_parts).
constexpr int kRoundParts = 4;
struct Bucket {
  flide_round_bufs bufs;
  flide_meta_layout L;
  hipGraph_t graph[kRoundParts] = {};
  hipGraphExec_t exec[kRoundParts] = {};
  Staging st;
  bool live = true;  // false once released: the id is never reused, replays of it are rejected
};

}  // namespace

struct flide_ctx {
  int device = 0;
  std::string err;
  int hip_err = 0;  // raw hipError_t behind the last FLIDE_E_HIP
  std::vector<RopeTable> ropes;
  std::vector<Bucket*> buckets;
  Staging direct;
  hipStream_t capture_stream = nullptr;
};

namespace {

flide_status fail(flide_ctx* ctx, flide_status st, const std::string& msg) {
  if (ctx) ctx->err = msg;
  return st;
}

flide_status fail_hip(flide_ctx* ctx, hipError_t e, const std::string& what) {
  if (ctx) ctx->hip_err = int(e);
  return fail(ctx, FLIDE_E_HIP, what + ": " + hipGetErrorString(e));
}

#define FLIDE_HIP(ctx, call)                              \
  do {                                                    \
    hipError_t e_ = (call);                               \
    if (e_ != hipSuccess) return fail_hip(ctx, e_, #call); \
  } while (0)

#define FLIDE_TRY(expr)                     \
  do {                                      \
    flide_status s_ = (expr);               \
    if (s_ != FLIDE_OK) return s_;          \
  } while (0)

flide_status launched(flide_ctx* ctx, int rc, const char* what) {
  if (rc != 0) return fail_hip(ctx, hipError_t(rc), what);
  return FLIDE_OK;
}

flide_status staging_init(flide_ctx* ctx, Staging& st, int64_t words) {
  if (st.words >= words) return FLIDE_OK;
  for (int i = 0; i < 2; ++i) {
    if (st.done[i]) {
      FLIDE_HIP(ctx, hipEventSynchronize(st.done[i]));
    }
    if (st.host[i]) {
      FLIDE_HIP(ctx, hipHostFree(st.host[i]));
      st.host[i] = nullptr;
    }
    FLIDE_HIP(ctx, hipHostMalloc((void**)&st.host[i], size_t(words) * sizeof(int32_t), hipHostMallocDefault));
    if (!st.done[i]) {
      FLIDE_HIP(ctx, hipEventCreateWithFlags(&st.done[i], hipEventDisableTiming));
    }
  }
  st.words = words;
  return FLIDE_OK;
}

void staging_free(Staging& st) {
  for (int i = 0; i < 2; ++i) {
    if (st.done[i]) {
      (void)hipEventSynchronize(st.done[i]);
      (void)hipEventDestroy(st.done[i]);
    }
    if (st.host[i]) (void)hipHostFree(st.host[i]);
    st.host[i] = nullptr;
    st.done[i] = nullptr;
  }
  st.words = 0;
}

void bucket_free(Bucket* b) {
  for (int i = 0; i < kRoundParts; ++i) {
    if (b->exec[i]) (void)hipGraphExecDestroy(b->exec[i]);
    if (b->graph[i]) (void)hipGraphDestroy(b->graph[i]);
    b->exec[i] = nullptr;
    b->graph[i] = nullptr;
  }
  staging_free(b->st);
  b->live = false;
}

// Copy `words` of `image` into the next pinned buffer (waiting until its
// previous copy has left it) and enqueue the H2D copy into `dst`.
flide_status staging_upload(flide_ctx* ctx, Staging& st, const int32_t* image, int64_t words, int32_t* dst,
                            hipStream_t stream) {
  FLIDE_TRY(staging_init(ctx, st, words));
  const int k = st.next;
  FLIDE_HIP(ctx, hipEventSynchronize(st.done[k]));
  std::memcpy(st.host[k], image, size_t(words) * sizeof(int32_t));
  FLIDE_HIP(ctx, hipMemcpyAsync(dst, st.host[k], size_t(words) * sizeof(int32_t), hipMemcpyHostToDevice, stream));
  FLIDE_HIP(ctx, hipEventRecord(st.done[k], stream));
  st.next = k ^ 1;
  return FLIDE_OK;
}

flide_status check_image(flide_ctx* ctx, const flide_caps& caps, const flide_meta_layout& L, const int32_t* img) {
  const int32_t* hdr = img + L.hdr;
  if (hdr[H_MAGIC] != kMagic) return fail(ctx, FLIDE_E_INVALID_ARG, "metadata image was not written by flide_plan_round");
  if (hdr[H_T] < 0 || hdr[H_T] > caps.T_cap || hdr[H_R] < 0 || hdr[H_R] > caps.R_cap || hdr[H_NQST] < 0 ||
      hdr[H_NQST] > caps.Q_cap || hdr[H_NSEG] != hdr[H_R] + hdr[H_NQST] || hdr[H_NTILES] < 0 ||
      hdr[H_NTILES] > L.tile_cap)
    return fail(ctx, FLIDE_E_CAPACITY, "metadata image does not fit the capacity");
  return FLIDE_OK;
}

// Rotary table [max_pos, d/2, 2] of (cos, sin) for angle t * theta^(-2i/d),
// evaluated in fp64 on the host and stored as fp32.
std::vector<float> rope_table_host(double theta, int d, int max_pos) {
  const int half = d / 2;
  std::vector<float> h(size_t(max_pos) * half * 2);
  for (int i = 0; i < half; ++i) {
    const double inv = std::pow(theta, -2.0 * double(i) / double(d));
    for (int p = 0; p < max_pos; ++p) {
      const double a = double(p) * inv;
      h[(size_t(p) * half + i) * 2] = float(std::cos(a));
      h[(size_t(p) * half + i) * 2 + 1] = float(std::sin(a));
    }
  }
  return h;
}

// A table of this context that covers (theta, d, max_pos), if any.
bool find_rope(const flide_ctx* ctx, double theta, int d, int max_pos, RopeArgs* out) {
  for (auto& t : ctx->ropes) {
    if (t.theta == theta && t.d == d && t.max_pos >= max_pos) {
      out->table = t.dev;
      out->max_pos = t.max_pos;
      return true;
    }
  }
  return false;
}

flide_status ensure_rope(flide_ctx* ctx, double theta, int d, int max_pos, RopeArgs* out) {
  if (find_rope(ctx, theta, d, max_pos, out)) return FLIDE_OK;
  std::vector<float> h = rope_table_host(theta, d, max_pos);
  float* dev = nullptr;
  FLIDE_HIP(ctx, hipMalloc((void**)&dev, h.size() * sizeof(float)));
  hipError_t e = hipMemcpy(dev, h.data(), h.size() * sizeof(float), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(dev);
    return fail_hip(ctx, e, "hipMemcpy(rope table)");
  }
  ctx->ropes.push_back({theta, d, max_pos, dev});
  out->table = dev;
  out->max_pos = max_pos;
  return FLIDE_OK;
}

flide_status check_attn(flide_ctx* ctx, const flide_attn_params* p) {
  if (!p) return fail(ctx, FLIDE_E_INVALID_ARG, "attention params are NULL");
  if (p->Hq < 1 || p->Hkv < 1 || p->Hq % p->Hkv != 0)
    return fail(ctx, FLIDE_E_INVALID_ARG, "need Hq, Hkv >= 1 and Hq % Hkv == 0");
  if (p->d < 8 || p->d > 256 || p->d % 8 != 0) return fail(ctx, FLIDE_E_UNSUPPORTED, "head size must be a multiple of 8 in [8, 256]");
  if (p->window < 0) return fail(ctx, FLIDE_E_INVALID_ARG, "window must be >= 0");
  if (p->max_pos < 1 || !(p->theta > 0.0)) return fail(ctx, FLIDE_E_INVALID_ARG, "need max_pos >= 1 and theta > 0");
  if (p->dtype != FLIDE_F32 && p->dtype != FLIDE_BF16) return fail(ctx, FLIDE_E_UNSUPPORTED, "dtype must be f32 or bf16");
  if (p->cache_rows < 0 || p->cache_slots < 0 || p->cache_rows % 8 != 0)
    return fail(ctx, FLIDE_E_INVALID_ARG, "cache shape must be >= 0 with cache_rows a multiple of 8");
  int64_t table_bytes = int64_t(p->max_pos) * p->d * 4;
  if (table_bytes > (int64_t(1) << 32)) return fail(ctx, FLIDE_E_UNSUPPORTED, "rotary table above 4 GiB");
  return FLIDE_OK;
}

flide_status check_gdn(flide_ctx* ctx, const flide_gdn_params* p, int32_t n_slots) {
  if (!p) return fail(ctx, FLIDE_E_INVALID_ARG, "GDN params are NULL");
  auto ok_dim = [](int v) { return v == 16 || v == 32 || v == 64 || v == 128; };
  if (p->H < 1 || !ok_dim(p->dk) || !ok_dim(p->dv))
    return fail(ctx, FLIDE_E_UNSUPPORTED, "GDN needs H >= 1 and dk, dv in {16, 32, 64, 128}");
  // the per-token kernel covers value blocks of min(dv, 32) channels for dk >= value block
  if (p->dk < (p->dv >= 32 ? 32 : p->dv))
    return fail(ctx, FLIDE_E_UNSUPPORTED, "GDN needs dk >= min(dv, 32)");
  if (p->conv_k < 1 || p->conv_k > 4) return fail(ctx, FLIDE_E_UNSUPPORTED, "conv width must be 1..4");
  if (p->act != 0 && p->act != 1) return fail(ctx, FLIDE_E_INVALID_ARG, "act must be 0 (none) or 1 (SiLU)");
  if (p->dtype != FLIDE_F32 && p->dtype != FLIDE_BF16) return fail(ctx, FLIDE_E_UNSUPPORTED, "dtype must be f32 or bf16");
  if (p->chunk != 0 && p->chunk != 64) return fail(ctx, FLIDE_E_UNSUPPORTED, "chunk must be 64 (or 0 for the default)");
  if (n_slots < 1) return fail(ctx, FLIDE_E_INVALID_ARG, "need at least one pool slot");
  return FLIDE_OK;
}

flide_status check_readout(flide_ctx* ctx, const flide_readout_params* p) {
  if (!p) return fail(ctx, FLIDE_E_INVALID_ARG, "readout params are NULL");
  if (p->hidden < 8 || p->hidden % 8 != 0 || p->hidden > 8192)
    return fail(ctx, FLIDE_E_UNSUPPORTED, "hidden must be a multiple of 8 in [8, 8192]");
  if (p->dtype != FLIDE_F32 && p->dtype != FLIDE_BF16) return fail(ctx, FLIDE_E_UNSUPPORTED, "dtype must be f32 or bf16");
  return FLIDE_OK;
}

flide_status view_of(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta, MetaView* mv,
                     flide_meta_layout* Lout = nullptr) {
  if (!caps || !dev_meta) return fail(ctx, FLIDE_E_INVALID_ARG, "caps or dev_meta is NULL");
  flide_meta_layout L;
  if (compute_layout(*caps, L) != FLIDE_OK) return fail(ctx, FLIDE_E_INVALID_ARG, "invalid capacity");
  *mv = make_view(const_cast<int32_t*>(dev_meta), L, *caps);
  if (Lout) *Lout = L;
  return FLIDE_OK;
}

flide_status enqueue_attn_prepare(flide_ctx* ctx, const MetaView& mv, const flide_attn_params& p, const void* k,
                                  const void* v, void* ws, hipStream_t stream) {
  if (!k || !v || !ws) return fail(ctx, FLIDE_E_INVALID_ARG, "attention buffer is NULL");
  RopeArgs rope;
  FLIDE_TRY(ensure_rope(ctx, p.theta, p.d, p.max_pos, &rope));
  return launched(ctx, launch_attn_prepare(mv, p, rope, k, v, ws, stream), "attn_prepare");
}

flide_status enqueue_attn_core(flide_ctx* ctx, const MetaView& mv, const flide_attn_params& p, const void* q,
                               const void* v, const void* kc, const void* vc, void* o, const void* ws,
                               hipStream_t stream) {
  if (!q || !v || !o || !ws) return fail(ctx, FLIDE_E_INVALID_ARG, "attention buffer is NULL");
  if (p.cache_rows > 0 && (!kc || !vc || p.cache_slots < 1))
    return fail(ctx, FLIDE_E_INVALID_ARG, "K/V cache shape given without cache buffers");
  RopeArgs rope;
  FLIDE_TRY(ensure_rope(ctx, p.theta, p.d, p.max_pos, &rope));
  return launched(ctx, launch_attn_core(mv, p, rope, q, v, p.cache_rows > 0 ? kc : nullptr,
                                        p.cache_rows > 0 ? vc : nullptr, o, ws, stream),
                  "attn_core");
}

// The attention layer over a given rotary table (no table is built here: nothing is allocated).
flide_status enqueue_attn_with(flide_ctx* ctx, const MetaView& mv, const flide_attn_params& p, const RopeArgs& rope,
                               const void* q, const void* k, const void* v, const void* kc, const void* vc, void* o,
                               void* ws, hipStream_t stream) {
  if (!q || !k || !v || !o || !ws) return fail(ctx, FLIDE_E_INVALID_ARG, "attention buffer is NULL");
  if (p.cache_rows > 0 && (!kc || !vc || p.cache_slots < 1))
    return fail(ctx, FLIDE_E_INVALID_ARG, "K/V cache shape given without cache buffers");
  FLIDE_TRY(launched(ctx, launch_attn_prepare(mv, p, rope, k, v, ws, stream), "attn_prepare"));
  return launched(ctx, launch_attn_core(mv, p, rope, q, v, p.cache_rows > 0 ? kc : nullptr,
                                        p.cache_rows > 0 ? vc : nullptr, o, ws, stream),
                  "attn_core");
}

flide_status enqueue_attn(flide_ctx* ctx, const MetaView& mv, const flide_attn_params& p, const void* q,
                          const void* k, const void* v, const void* kc, const void* vc, void* o, void* ws,
                          hipStream_t stream) {
  if (!q || !o) return fail(ctx, FLIDE_E_INVALID_ARG, "attention buffer is NULL");
  FLIDE_TRY(enqueue_attn_prepare(ctx, mv, p, k, v, ws, stream));
  return enqueue_attn_core(ctx, mv, p, q, v, kc, vc, o, ws, stream);
}

flide_status enqueue_gdn(flide_ctx* ctx, const MetaView& mv, const flide_gdn_params& p, int phase, const void* x,
                         const float* conv_w, const float* alpha, const float* eta, float* state_pool,
                         void* conv_pool, int32_t n_slots, void* o, hipStream_t stream) {
  if (!x || !conv_w || !alpha || !eta || !state_pool || !o || (p.conv_k > 1 && !conv_pool))
    return fail(ctx, FLIDE_E_INVALID_ARG, "GDN buffer is NULL");
  if (phase != 0 && phase != 1) return fail(ctx, FLIDE_E_INVALID_ARG, "phase must be 0 (trunks) or 1 (questions)");
  return launched(ctx, launch_gdn(mv, p, phase, x, conv_w, alpha, eta, state_pool, conv_pool, n_slots, o, stream),
                  "fork_gdn");
}

// One part of a round (the parts of a captured bucket, in order):
//   0  metadata expansion (reads the uploaded image, writes the per-row and per-tile metadata);
//   1  GDN call 1, trunks (writes the trunk states, windows and outputs);
//   2  attention and interior checkpoint K/V (reads the expanded metadata and the round's q, k, v);
//   3  GDN call 2, questions (reads part 1's states by slot index), then the readout.
flide_status enqueue_round_part(flide_ctx* ctx, const flide_round_bufs* b, int part, hipStream_t stream) {
  MetaView mv;
  FLIDE_TRY(view_of(ctx, &b->caps, b->dev_meta, &mv));
  if (part == 0) return launched(ctx, launch_meta_expand(mv, stream), "meta_expand");
  if (part == 1 || part == 3) {
    FLIDE_TRY(enqueue_gdn(ctx, mv, b->gdn, part == 1 ? 0 : 1, b->x, b->conv_w, b->alpha, b->eta, b->state_pool,
                          b->conv_pool, b->n_slots, b->o_gdn, stream));
    if (part == 1) return FLIDE_OK;
    if (!b->h || !b->w_opt || !b->opt_off || !b->opt_id || !b->probs)
      return fail(ctx, FLIDE_E_INVALID_ARG, "readout buffer is NULL");
    return launched(ctx, launch_readout(mv, b->ro, b->h, b->w_opt, b->opt_off, b->opt_id, b->n_opt_rows, b->probs,
                                        stream),
                    "readout");
  }
  for (int l = 0; l < b->n_attn; ++l) {
    const flide_attn_params& ap = b->attn[l];
    FLIDE_TRY(enqueue_attn(ctx, mv, ap, b->q[l], b->k[l], b->v[l], b->k_cache[l], b->v_cache[l], b->o_attn[l],
                           b->attn_ws[l], stream));
    // interior checkpoints of the round (requests with save_m > 0): their K/V go to the cache slot
    // from the workspace the prepare step just wrote; requests without one exit at once
    if (ap.cache_rows > 0 && b->k_cache[l] && b->v_cache[l])
      FLIDE_TRY(launched(ctx,
                         launch_attn_save_kv(mv, ap, b->v[l], b->attn_ws[l], const_cast<void*>(b->k_cache[l]),
                                             const_cast<void*>(b->v_cache[l]), stream),
                         "attn_save_kv"));
  }
  return FLIDE_OK;
}

flide_status enqueue_round(flide_ctx* ctx, const flide_round_bufs* b, hipStream_t stream) {
  for (int part = 0; part < kRoundParts; ++part) FLIDE_TRY(enqueue_round_part(ctx, b, part, stream));
  return FLIDE_OK;
}

flide_status check_round_bufs(flide_ctx* ctx, const flide_round_bufs* b) {
  if (!b) return fail(ctx, FLIDE_E_INVALID_ARG, "round buffers are NULL");
  flide_meta_layout L;
  if (compute_layout(b->caps, L) != FLIDE_OK) return fail(ctx, FLIDE_E_INVALID_ARG, "invalid capacity");
  if (!b->dev_meta) return fail(ctx, FLIDE_E_INVALID_ARG, "dev_meta is NULL");
  if (b->n_attn < 0 || b->n_attn > 2) return fail(ctx, FLIDE_E_INVALID_ARG, "n_attn must be 0, 1 or 2");
  for (int l = 0; l < b->n_attn; ++l) FLIDE_TRY(check_attn(ctx, &b->attn[l]));
  FLIDE_TRY(check_gdn(ctx, &b->gdn, b->n_slots));
  FLIDE_TRY(check_readout(ctx, &b->ro));
  return FLIDE_OK;
}

// parts: bit i replays part i (in part order); part 0 uploads `image` first
flide_status graph_replay_parts(flide_ctx* ctx, int32_t bucket_id, const int32_t* image, void* stream, int parts) {
  if (parts <= 0 || parts >= (1 << kRoundParts)) return fail(ctx, FLIDE_E_INVALID_ARG, "parts must be a mask of 1 .. 15");
  if (bucket_id < 0 || size_t(bucket_id) >= ctx->buckets.size() || !ctx->buckets[size_t(bucket_id)]->live)
    return fail(ctx, FLIDE_E_INVALID_ARG, "no such bucket (never captured, or released)");
  Bucket* b = ctx->buckets[size_t(bucket_id)];
  FLIDE_HIP(ctx, hipSetDevice(ctx->device));
  if (parts & 1) {
    if (!image) return fail(ctx, FLIDE_E_INVALID_ARG, "image is NULL");
    FLIDE_TRY(check_image(ctx, b->bufs.caps, b->L, image));
    FLIDE_TRY(staging_upload(ctx, b->st, image, b->L.host_words, b->bufs.dev_meta, (hipStream_t)stream));
  }
  for (int part = 0; part < kRoundParts; ++part)
    if (parts & (1 << part)) FLIDE_HIP(ctx, hipGraphLaunch(b->exec[part], (hipStream_t)stream));
  return FLIDE_OK;
}

}  // namespace

extern "C" {

flide_status flide_create(flide_ctx** out, int32_t device) {
  if (!out) return FLIDE_E_INVALID_ARG;
  *out = nullptr;
  try {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return FLIDE_E_HIP;
    if (hipSetDevice(device) != hipSuccess) return FLIDE_E_HIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return FLIDE_E_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return FLIDE_E_UNSUPPORTED;
    // the allocation-free entry point's device scratch: its address on this GPU, taken once
    if (noalloc_scratch_init(device) != int(hipSuccess)) return FLIDE_E_HIP;
    flide_ctx* ctx = new flide_ctx();
    ctx->device = device;
    if (hipStreamCreateWithFlags(&ctx->capture_stream, hipStreamNonBlocking) != hipSuccess) {
      delete ctx;
      return FLIDE_E_HIP;
    }
    *out = ctx;
    return FLIDE_OK;
  } catch (...) {
    return FLIDE_E_INTERNAL;
  }
}

void flide_destroy(flide_ctx* ctx) {
  if (!ctx) return;
  (void)hipSetDevice(ctx->device);
  (void)hipDeviceSynchronize();
  for (Bucket* b : ctx->buckets) {
    bucket_free(b);
    delete b;
  }
  staging_free(ctx->direct);
  for (auto& t : ctx->ropes) (void)hipFree(t.dev);
  if (ctx->capture_stream) (void)hipStreamDestroy(ctx->capture_stream);
  delete ctx;
}

const char* flide_last_error(const flide_ctx* ctx) { return ctx ? ctx->err.c_str() : ""; }

int32_t flide_last_hip_error(const flide_ctx* ctx) { return ctx ? ctx->hip_err : 0; }

flide_status flide_meta_upload(flide_ctx* ctx, const flide_caps* caps, const int32_t* image, int32_t* dev_meta,
                               void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    if (!image) return fail(ctx, FLIDE_E_INVALID_ARG, "image is NULL");
    MetaView mv;
    flide_meta_layout L;
    FLIDE_TRY(view_of(ctx, caps, dev_meta, &mv, &L));
    FLIDE_TRY(check_image(ctx, *caps, L, image));
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    FLIDE_TRY(staging_upload(ctx, ctx->direct, image, L.host_words, dev_meta, (hipStream_t)stream));
    return launched(ctx, launch_meta_expand(mv, stream), "meta_expand");
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_meta_upload");
  }
}

flide_status flide_attn_workspace_bytes(const flide_caps* caps, const flide_attn_params* p, int64_t* bytes) {
  if (!caps || !p || !bytes) return FLIDE_E_INVALID_ARG;
  if (caps->T_cap < 1 || p->Hkv < 1 || p->d < 1) return FLIDE_E_INVALID_ARG;
  *bytes = attn_workspace_bytes(*caps, *p);
  return FLIDE_OK;
}

flide_status flide_fork_attn(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta,
                             const flide_attn_params* p, const void* q, const void* k, const void* v,
                             const void* k_cache, const void* v_cache, void* o, void* workspace, void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    FLIDE_TRY(check_attn(ctx, p));
    MetaView mv;
    FLIDE_TRY(view_of(ctx, caps, dev_meta, &mv));
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    return enqueue_attn(ctx, mv, *p, q, k, v, k_cache, v_cache, o, workspace, (hipStream_t)stream);
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_fork_attn");
  }
}

flide_status flide_fork_attn_noalloc(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta,
                                     const flide_attn_params* p, const void* q, const void* k, const void* v,
                                     const void* k_cache, const void* v_cache, void* o, void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    FLIDE_TRY(check_attn(ctx, p));
    MetaView mv;
    FLIDE_TRY(view_of(ctx, caps, dev_meta, &mv));
    const int64_t need = attn_workspace_bytes(*caps, *p);
    if (need > kNoAllocWorkspaceBytes)
      return fail(ctx, FLIDE_E_CAPACITY,
                  "flide_fork_attn_noalloc: these capacities need " + std::to_string(need) +
                      " bytes of attention workspace; the library's scratch holds " +
                      std::to_string(kNoAllocWorkspaceBytes) + " (use flide_fork_attn with a workspace)");
    void* ws = noalloc_workspace(ctx->device);
    if (!ws) return fail(ctx, FLIDE_E_INTERNAL, "device scratch was not set up");
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    RopeArgs rope;
    if (!find_rope(ctx, p->theta, p->d, p->max_pos, &rope)) {
      // no table of this context covers the call: use the scratch's table region, written from the same
      // host fp64 evaluation as every other table when it does not already hold these parameters
      const int64_t tbytes = int64_t(p->max_pos) * p->d * 4;
      if (tbytes > kNoAllocTableBytes)
        return fail(ctx, FLIDE_E_CAPACITY,
                    "flide_fork_attn_noalloc: a rotary table of " + std::to_string(tbytes) +
                        " bytes does not fit the library's scratch (" + std::to_string(kNoAllocTableBytes) + ")");
      bool holds = false;
      float* table = noalloc_table(ctx->device, p->theta, p->d, p->max_pos, &holds, false);
      if (!table) return fail(ctx, FLIDE_E_INTERNAL, "device scratch was not set up");
      if (!holds) {
        std::vector<float> h = rope_table_host(p->theta, p->d, p->max_pos);
        FLIDE_HIP(ctx, hipMemcpyAsync(table, h.data(), h.size() * sizeof(float), hipMemcpyHostToDevice,
                                      (hipStream_t)stream));
        FLIDE_HIP(ctx, hipStreamSynchronize((hipStream_t)stream));  // the host copy is freed on return
        noalloc_table(ctx->device, p->theta, p->d, p->max_pos, &holds, true);
      }
      rope.table = table;
      rope.max_pos = p->max_pos;
    }
    return enqueue_attn_with(ctx, mv, *p, rope, q, k, v, k_cache, v_cache, o, ws, (hipStream_t)stream);
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_fork_attn_noalloc");
  }
}

flide_status flide_attn_prepare(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta,
                                const flide_attn_params* p, const void* k, const void* v, void* workspace,
                                void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    FLIDE_TRY(check_attn(ctx, p));
    MetaView mv;
    FLIDE_TRY(view_of(ctx, caps, dev_meta, &mv));
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    return enqueue_attn_prepare(ctx, mv, *p, k, v, workspace, (hipStream_t)stream);
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_attn_prepare");
  }
}

flide_status flide_attn_save_kv(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta,
                                const flide_attn_params* p, const void* v, const void* workspace, void* k_cache,
                                void* v_cache, void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    FLIDE_TRY(check_attn(ctx, p));
    if (!v || !workspace || !k_cache || !v_cache || p->cache_rows < 1 || p->cache_slots < 1)
      return fail(ctx, FLIDE_E_INVALID_ARG, "checkpoint K/V needs v, the workspace and a K/V cache");
    MetaView mv;
    FLIDE_TRY(view_of(ctx, caps, dev_meta, &mv));
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    return launched(ctx, launch_attn_save_kv(mv, *p, v, workspace, k_cache, v_cache, stream), "attn_save_kv");
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_attn_save_kv");
  }
}

flide_status flide_attn_core(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta,
                             const flide_attn_params* p, const void* q, const void* v, const void* k_cache,
                             const void* v_cache, void* o, const void* workspace, void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    FLIDE_TRY(check_attn(ctx, p));
    MetaView mv;
    FLIDE_TRY(view_of(ctx, caps, dev_meta, &mv));
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    return enqueue_attn_core(ctx, mv, *p, q, v, k_cache, v_cache, o, workspace, (hipStream_t)stream);
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_attn_core");
  }
}

flide_status flide_fork_gdn(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta,
                            const flide_gdn_params* p, int32_t phase, const void* x, const float* conv_w,
                            const float* alpha, const float* eta, float* state_pool, void* conv_pool,
                            int32_t n_slots, void* o, void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    FLIDE_TRY(check_gdn(ctx, p, n_slots));
    MetaView mv;
    FLIDE_TRY(view_of(ctx, caps, dev_meta, &mv));
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    return enqueue_gdn(ctx, mv, *p, phase, x, conv_w, alpha, eta, state_pool, conv_pool, n_slots, o,
                       (hipStream_t)stream);
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_fork_gdn");
  }
}

flide_status flide_readout(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta,
                           const flide_readout_params* p, const void* h, const void* w_opt,
                           const int32_t* opt_off, const int32_t* opt_id, int32_t n_opt_rows, float* probs,
                           void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    FLIDE_TRY(check_readout(ctx, p));
    if (!h || !w_opt || !opt_off || !opt_id || !probs) return fail(ctx, FLIDE_E_INVALID_ARG, "readout buffer is NULL");
    MetaView mv;
    FLIDE_TRY(view_of(ctx, caps, dev_meta, &mv));
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    return launched(ctx, launch_readout(mv, *p, h, w_opt, opt_off, opt_id, n_opt_rows, probs, stream), "readout");
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_readout");
  }
}

namespace {

flide_status check_rows(flide_ctx* ctx, int32_t rows, int32_t dtype) {
  if (rows != FLIDE_ROWS_ALL && rows != FLIDE_ROWS_QFINAL)
    return fail(ctx, FLIDE_E_INVALID_ARG, "rows must be FLIDE_ROWS_ALL or FLIDE_ROWS_QFINAL");
  if (dtype != FLIDE_F32 && dtype != FLIDE_BF16) return fail(ctx, FLIDE_E_UNSUPPORTED, "dtype must be f32 or bf16");
  return FLIDE_OK;
}

}  // namespace

flide_status flide_rmsnorm(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta, int32_t rows,
                           int32_t dtype, int32_t D, const void* x, const float* g, float eps, void* y,
                           void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    FLIDE_TRY(check_rows(ctx, rows, dtype));
    if (D < 1 || !x || !g || !y || !(eps >= 0.f)) return fail(ctx, FLIDE_E_INVALID_ARG, "rmsnorm: bad arguments");
    MetaView mv;
    FLIDE_TRY(view_of(ctx, caps, dev_meta, &mv));
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    return launched(ctx, launch_rmsnorm(mv, rows, dtype, D, x, g, eps, y, stream), "rmsnorm");
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_rmsnorm");
  }
}

flide_status flide_linear(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta, int32_t rows,
                          int32_t dtype, int32_t N, int32_t K, const void* a, int64_t lda, const void* w,
                          const void* resid, void* c, int64_t ldc, void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    FLIDE_TRY(check_rows(ctx, rows, dtype));
    if (N < 1 || K < 1 || !a || !w || !c || lda < K || ldc < N)
      return fail(ctx, FLIDE_E_INVALID_ARG, "linear: bad arguments");
    if (dtype == FLIDE_BF16 && (K % 32 != 0 || lda % 8 != 0))
      return fail(ctx, FLIDE_E_UNSUPPORTED, "linear (bf16): K must be a multiple of 32 and lda of 8");
    if (a == c) return fail(ctx, FLIDE_E_INVALID_ARG, "linear: the output must not alias the input rows");
    MetaView mv;
    FLIDE_TRY(view_of(ctx, caps, dev_meta, &mv));
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    return launched(ctx, launch_linear(mv, rows, dtype, N, K, a, lda, w, resid, c, ldc, stream), "linear");
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_linear");
  }
}

flide_status flide_swiglu(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta, int32_t rows,
                          int32_t dtype, int32_t F, const void* gu, void* out, void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    FLIDE_TRY(check_rows(ctx, rows, dtype));
    if (F < 1 || !gu || !out || gu == out) return fail(ctx, FLIDE_E_INVALID_ARG, "swiglu: bad arguments");
    MetaView mv;
    FLIDE_TRY(view_of(ctx, caps, dev_meta, &mv));
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    return launched(ctx, launch_swiglu(mv, rows, dtype, F, gu, out, stream), "swiglu");
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_swiglu");
  }
}

flide_status flide_gdn_gates(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta, int32_t dtype,
                             int32_t H, const void* z, const float* bias, float* alpha, float* eta, void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    FLIDE_TRY(check_rows(ctx, FLIDE_ROWS_ALL, dtype));
    if (H < 1 || !z || !bias || !alpha || !eta) return fail(ctx, FLIDE_E_INVALID_ARG, "gdn_gates: bad arguments");
    MetaView mv;
    FLIDE_TRY(view_of(ctx, caps, dev_meta, &mv));
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    return launched(ctx, launch_gates(mv, dtype, H, z, bias, alpha, eta, stream), "gdn_gates");
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_gdn_gates");
  }
}

flide_status flide_graph_capture(flide_ctx* ctx, const flide_round_bufs* bufs, void* stream, int32_t* bucket_id) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  (void)stream;
  try {
    if (!bucket_id) return fail(ctx, FLIDE_E_INVALID_ARG, "bucket_id is NULL");
    FLIDE_TRY(check_round_bufs(ctx, bufs));
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    // rotary tables are built before capture (their upload is not a graph node)
    for (int l = 0; l < bufs->n_attn; ++l) {
      RopeArgs r;
      FLIDE_TRY(ensure_rope(ctx, bufs->attn[l].theta, bufs->attn[l].d, bufs->attn[l].max_pos, &r));
    }
    Bucket* b = new Bucket();
    b->bufs = *bufs;
    compute_layout(bufs->caps, b->L);
    hipStream_t cs = ctx->capture_stream;
    for (int part = 0; part < kRoundParts; ++part) {
      hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
      if (e != hipSuccess) {
        bucket_free(b);
        delete b;
        return fail_hip(ctx, e, "hipStreamBeginCapture");
      }
      flide_status st = enqueue_round_part(ctx, bufs, part, cs);
      hipGraph_t g = nullptr;
      e = hipStreamEndCapture(cs, &g);
      if (st != FLIDE_OK || e != hipSuccess) {
        if (g) (void)hipGraphDestroy(g);
        bucket_free(b);
        delete b;
        if (st != FLIDE_OK) return st;
        return fail_hip(ctx, e, "hipStreamEndCapture");
      }
      b->graph[part] = g;
      e = hipGraphInstantiate(&b->exec[part], g, nullptr, nullptr, 0);
      if (e != hipSuccess) {
        bucket_free(b);
        delete b;
        return fail_hip(ctx, e, "hipGraphInstantiate");
      }
    }
    flide_status st = staging_init(ctx, b->st, b->L.host_words);
    if (st != FLIDE_OK) {
      bucket_free(b);
      delete b;
      return st;
    }
    ctx->buckets.push_back(b);
    *bucket_id = int32_t(ctx->buckets.size() - 1);
    return FLIDE_OK;
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_graph_capture");
  }
}

flide_status flide_select_bucket(const flide_ctx* ctx, int32_t T, int32_t R, int32_t n_q, int32_t* bucket_id) {
  if (!ctx || !bucket_id) return FLIDE_E_INVALID_ARG;
  int best = -1;
  for (size_t i = 0; i < ctx->buckets.size(); ++i) {
    if (!ctx->buckets[i]->live) continue;
    const flide_caps& c = ctx->buckets[i]->bufs.caps;
    if (c.T_cap >= T && c.R_cap >= R && c.Q_cap >= n_q) {
      if (best < 0 || c.T_cap < ctx->buckets[size_t(best)]->bufs.caps.T_cap) best = int(i);
    }
  }
  if (best < 0) return FLIDE_E_CAPACITY;
  *bucket_id = best;
  return FLIDE_OK;
}


flide_status flide_graph_replay(flide_ctx* ctx, int32_t bucket_id, const int32_t* image, void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    return graph_replay_parts(ctx, bucket_id, image, stream, 15);
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_graph_replay");
  }
}

flide_status flide_graph_replay_front(flide_ctx* ctx, int32_t bucket_id, const int32_t* image, void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    return graph_replay_parts(ctx, bucket_id, image, stream, 3);
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_graph_replay_front");
  }
}

flide_status flide_graph_replay_back(flide_ctx* ctx, int32_t bucket_id, void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    return graph_replay_parts(ctx, bucket_id, nullptr, stream, 12);
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_graph_replay_back");
  }
}

flide_status flide_graph_replay_parts(flide_ctx* ctx, int32_t bucket_id, const int32_t* image, int32_t parts,
                                     void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    return graph_replay_parts(ctx, bucket_id, image, stream, parts);
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_graph_replay_parts");
  }
}

flide_status flide_graph_release(flide_ctx* ctx, int32_t bucket_id) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    if (bucket_id < 0 || size_t(bucket_id) >= ctx->buckets.size() || !ctx->buckets[size_t(bucket_id)]->live)
      return fail(ctx, FLIDE_E_INVALID_ARG, "no such bucket (never captured, or released)");
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    // a replay still in flight holds the graph and the staging: wait for the device first
    FLIDE_HIP(ctx, hipDeviceSynchronize());
    bucket_free(ctx->buckets[size_t(bucket_id)]);
    return FLIDE_OK;
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_graph_release");
  }
}

flide_status flide_round_eager(flide_ctx* ctx, const flide_round_bufs* bufs, const int32_t* image, void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    FLIDE_TRY(check_round_bufs(ctx, bufs));
    if (!image) return fail(ctx, FLIDE_E_INVALID_ARG, "image is NULL");
    flide_meta_layout L;
    compute_layout(bufs->caps, L);
    FLIDE_TRY(check_image(ctx, bufs->caps, L, image));
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    FLIDE_TRY(staging_upload(ctx, ctx->direct, image, L.host_words, bufs->dev_meta, (hipStream_t)stream));
    return enqueue_round(ctx, bufs, (hipStream_t)stream);
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_round_eager");
  }
}

flide_status flide_check_device(flide_ctx* ctx, const flide_caps* caps, int32_t* dev_meta, void* stream) {
  if (!ctx) return FLIDE_E_INVALID_ARG;
  try {
    MetaView mv;
    FLIDE_TRY(view_of(ctx, caps, dev_meta, &mv));
    FLIDE_HIP(ctx, hipSetDevice(ctx->device));
    FLIDE_HIP(ctx, hipStreamSynchronize((hipStream_t)stream));
    int32_t err[4] = {0, 0, 0, 0};
    FLIDE_HIP(ctx, hipMemcpy(err, mv.dev_error, sizeof(err), hipMemcpyDeviceToHost));
    if (err[0] == 0) return FLIDE_OK;
    FLIDE_HIP(ctx, hipMemset(mv.dev_error, 0, sizeof(err)));
    char msg[160];
    std::snprintf(msg, sizeof(msg),
                  "device metadata check failed (bits 0x%x: 1 header, 2 position, 4 slot, 8 option, 16 cache, "
                  "32 segment)",
                  unsigned(err[0]));
    return fail(ctx, FLIDE_E_DEVICE, msg);
  } catch (...) {
    return fail(ctx, FLIDE_E_INTERNAL, "exception in flide_check_device");
  }
}

}  // extern "C"
