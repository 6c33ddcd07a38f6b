/*
 * flide.h — C ABI of the ForkAttention hot path for one MI355X (gfx950).
 *
 * One round of decision requests (a shared trunk s of P tokens plus questions
 * q_1..q_n per request) is executed as one flat, padding-free token stream
 * whose tree structure lives in device-resident metadata.  Sources, cited by
 * page title and section:
 *
 *  [ZH] "Flide: Accelerating Decision Inference with Exact State Forking"
 *       (paper.rainbus.top/paper/2610.42148): §前置知识 (Eq. (1), the gated
 *       delta rule), §核心方法 (flat stream, (j, c, t) metadata, two-call GDN,
 *       graphs bucketed by stream length T), §方法步骤详情 (stream order,
 *       visibility rule, sliding window, conv tail read by index, capacity
 *       split, selective readout, checkpoints at m).
 *  [KO] "Flide는 공유 상태를 정확히 분기해 결정 추론을 최대 9.5배 빠르게 한다"
 *       (onedev.kr/papers/1551): §어떻게 동작하나 (problem, Eq. (1)),
 *       §무엇과 다른가 (positions continue from P, Proposition 3.1),
 *       §어떻게 쓰나 (flat-graph execution, tail-only padding, request-boundary
 *       splitting, eager path for one oversized request, checkpoints,
 *       deterministic mode).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every function returns a flide_status; no C++ exception crosses the ABI.
 *  - Host-side validation runs before anything is enqueued: on an error
 *    nothing is launched and no caller memory is written.
 *  - "host" pointers point to CPU memory, "device" pointers to memory on the
 *    context's GPU.  The caller owns every buffer it passes; the library owns
 *    only what hangs off a flide_ctx (pinned staging, rotary tables, graphs).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    device work is stream ordered and asynchronous; only flide_check_device
 *    synchronises.
 *  - Outputs must not alias inputs.
 *  - One host thread at a time per flide_ctx.
 *
 * Stream layout (Flide summary [ZH] §方法步骤详情): all trunks in request
 * order, then all questions grouped by request, in question order.  Row
 * metadata (j, c, t): request, branch (0 = trunk, i = question i, 1-based),
 * position; question positions continue from P ([KO] §무엇과 다른가).  Rows
 * past T up to the capacity are tail padding with (j, c, t) = (-1, -1, -1);
 * kernels leave their outputs untouched.
 */
#ifndef FLIDE_H
#define FLIDE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLIDE_OK = 0,
  FLIDE_E_INVALID_ARG = 1, /* a host-side check failed; nothing was enqueued        */
  FLIDE_E_CAPACITY = 2,    /* the round does not fit the capacity / no bucket fits  */
  FLIDE_E_UNSUPPORTED = 3, /* a shape or dtype the kernels do not implement         */
  FLIDE_E_HIP = 4,         /* a HIP runtime call failed (see flide_last_error)      */
  FLIDE_E_DEVICE = 5,      /* a device-side metadata check tripped                  */
  FLIDE_E_INTERNAL = 6     /* unexpected failure inside the library                 */
} flide_status;

typedef enum { FLIDE_F32 = 0, FLIDE_BF16 = 1 } flide_dtype;

typedef struct flide_ctx flide_ctx;

/* Infrastructure (no passage of the pages defines error reporting).
 * Static description of the status code (never NULL). */
const char* flide_status_string(int32_t status);
/* Infrastructure.  Library version string (never NULL). */
const char* flide_version(void);

/* ------------------------------------------------------------------------
 * Requests and capacities (host structures)
 * ------------------------------------------------------------------------ */

/* One decision request r = (s, q_1..q_n) ([KO] §어떻게 동작하나).
 *  P         trunk length including any checkpointed prefix, >= 0
 *  m         resume position, 0 <= m <= P; the stream holds trunk positions m..P-1
 *            (checkpoint resume, [KO] §어떻게 쓰나)
 *  n_q       number of questions, >= 0
 *  q_len     host array of n_q lengths, each >= 1 (may be NULL when n_q == 0)
 *  ckpt_slot pool slot holding the checkpoint at m (GDN state, conv window,
 *            attention K/V of positions 0..m-1); required when m > 0, else -1
 *  out_slot  pool slot that receives S_P and the conv window after the trunk,
 *            >= 0 and != ckpt_slot when m > 0
 *  save_m    0, or a checkpoint to create at trunk position save_m in the same
 *            pass (the interior checkpoints that a later round resumes from,
 *            [KO] §어떻게 쓰나): m < save_m <= P, and save_m - m a multiple of
 *            64 (a chunk boundary of the trunk) unless save_m == P
 *  save_slot pool slot that receives the GDN state after position save_m - 1
 *            and the conv window of positions save_m - conv_k + 1 .. save_m - 1
 *            (flide_fork_gdn, phase 0), and the attention K/V of positions
 *            0..save_m-1 (flide_attn_save_kv); -1 when save_m == 0.  Distinct
 *            from every out_slot, ckpt_slot and save_slot of the round.        */
typedef struct {
  int32_t P;
  int32_t m;
  int32_t n_q;
  const int32_t* q_len;
  int32_t ckpt_slot;
  int32_t out_slot;
  int32_t save_m;
  int32_t save_slot;
} flide_request;

/* Capacity of a metadata image / graph bucket: stream rows, requests, questions. */
typedef struct {
  int32_t T_cap;
  int32_t R_cap;
  int32_t Q_cap;
} flide_caps;

/* Word offsets (int32 units) of the arrays inside a metadata image.  The first
 * `host_words` words are written by flide_plan_round and uploaded as is; the
 * per-row arrays tok_j/tok_c/tok_t and the device error words are filled on the
 * device.  Segments are ordered trunks first (index j = request j), then
 * questions in stream order.
 *   hdr[0..15]  T, R, n_seg, n_qst, n_tiles, max_pos, tile_group, 0..., magic  (tile_group: attention
 *               work order, 0 = every head group of a tile position in turn, n = runs of n positions
 *               per head group; chosen by the planner for rounds whose tiles see thousands of keys)
 *   seg_*       [seg_cap]  row0, len, req, branch, pos0, state (slot or -1),
 *                          vcol0: column offset of the segment in the transposed
 *                          value workspace (column = vcol0 + position, congruent
 *                          to the position modulo 32: 32-aligned positions start a
 *                          column block of the tile-major workspace)
 *   req_*       [R_cap]    trunk_row0, P, m, ckpt_slot, out_slot, q_seg0, n_q,
 *                          save_m, save_slot (0 and -1 when no checkpoint is made)
 *   qfin_row    [Q_cap]    last stream row of every question (stream order)
 *   tile_seg    [tile_cap * 4] attention work list: a tile is four units of up
 *                          to 8 rows; unit u of position x is at x * 4 + u:
 *                          its segment (-1: no unit; unit 0 of a used position
 *                          always exists) ...
 *   tile_row0   [tile_cap * 4] ... and its first stream row.  A tile's units
 *                          are consecutive rows of one trunk, or rows of up to
 *                          four questions of one request
 *   tile_swa    [tile_cap] the windowed layer's order of the same work list:
 *                          entry i is the position its i-th workgroup (per
 *                          head group) takes, -1 for none
 *   gdn_order   [seg_cap]  GDN work list: trunk segments, then question segments,
 *                          each by length, longest first (ties in stream order)
 *   tok_j/c/t   [T_cap]    per-row metadata (device only)
 *   tile_desc   [tile_cap * 48] per attention work-list position: segment of
 *                          unit 0 (-1 if unused), question flag, P, m, checkpoint
 *                          slot, key-row and value-column offsets of the trunk,
 *                          first and last query position, own ranges; per unit:
 *                          first row, rows, first position, own range; per own
 *                          range (a segment among the units): key-row and
 *                          value-column offsets, first and one-past-last position
 *                          (device only)
 *   dev_error   [4]        device error word (device only)                     */
typedef struct {
  int64_t host_words;
  int64_t dev_words;
  int64_t hdr;
  int64_t seg_row0, seg_len, seg_req, seg_branch, seg_pos0, seg_state, seg_vcol0;
  int64_t req_trunk_row0, req_P, req_m, req_ckpt, req_out, req_q_seg0, req_nq, req_save_m, req_save_slot;
  int64_t qfin_row;
  int64_t tile_seg, tile_row0, tile_swa;
  int64_t gdn_order;
  int64_t tok_j, tok_c, tok_t;
  int64_t tile_desc;
  int64_t dev_error;
  int32_t seg_cap;
  int32_t tile_cap;
  int32_t tile_rows; /* query rows per attention tile */
  int32_t reserved;
} flide_meta_layout;

/* Offsets and sizes of a metadata image for `caps` (host only, no GPU needed): the
 * device buffers of segment lengths, positions, key ranges and state indices that
 * each round rewrites before its graph replay ([ZH] §方法步骤详情 third step;
 * [KO] §어떻게 쓰나).  out (host) is written on success only.
 * Errors: FLIDE_E_INVALID_ARG for NULL pointers or capacities < 1 or too large. */
flide_status flide_meta_layout_for(const flide_caps* caps, flide_meta_layout* out);

/* Stream rows T, segments and questions a round needs (host only): T is the
 * padding-free stream length P - m + sum |q_i| summed over the requests, the
 * P + sum |q_i| work of [KO] §어떻게 동작하나 (minus any checkpointed prefix).
 * T, n_seg, n_qst (host, each may be NULL) are written on success only.
 * Errors: FLIDE_E_INVALID_ARG for an invalid request (m > P, |q| < 1, m > 0
 * without a checkpoint slot, negative sizes, ...).                            */
flide_status flide_plan_sizes(const flide_request* reqs, int32_t R, int32_t* T, int32_t* n_seg,
                              int32_t* n_qst);

/* Host planner ([ZH] §方法步骤详情 first step; [KO] §어떻게 쓰나): writes the
 * metadata image of the round into `image` (host, `image_words` >= host_words
 * of the layout for `caps`).  Segment lengths, positions, key ranges (via the
 * request table) and state indices; the attention tile list; question-final
 * rows.  Errors: FLIDE_E_INVALID_ARG (bad request), FLIDE_E_CAPACITY (T, R or
 * the number of questions exceeds `caps`).  `image` is untouched on error.     */
flide_status flide_plan_round(const flide_request* reqs, int32_t R, const flide_caps* caps, int32_t* image,
                              int64_t image_words);

/* Request-boundary split ([KO] §어떻게 쓰나; [ZH] §方法步骤详情 third step):
 * greedy in request order, at most T_max rows per sub-round; a request with
 * more than T_max rows is a sub-round of its own flagged eager (run without a
 * graph).  sub_first (host, R+1 entries) receives the first request of every
 * sub-round plus a final R; eager (host, R entries) one flag per sub-round;
 * *n_sub the number of sub-rounds.  Errors: FLIDE_E_INVALID_ARG.              */
flide_status flide_split_round(const flide_request* reqs, int32_t R, int32_t T_max, int32_t* sub_first,
                               int32_t* n_sub, uint8_t* eager);

/* ------------------------------------------------------------------------
 * Prefix-match checkpoint store (host only, no GPU needed)
 * ------------------------------------------------------------------------
 * A request may resume at m from a checkpoint only if its tokens match the
 * checkpoint's up to m ([KO] §어떻게 쓰나).  The library never sees tokens: the
 * caller names a prefix by a 64-bit digest of its first m tokens (any hash it
 * likes; equal digests are taken as equal prefixes).  The store manages the
 * pool slots [first_slot, first_slot + n_slots) of the state, conv and K/V
 * pools: it maps (m, digest) to the slot holding that checkpoint, hands out
 * slots for new checkpoints (free ones first, else evicting the least
 * recently used committed entry that no round holds), and keeps a reference
 * count per slot so that a slot a round reads or writes is never evicted.
 * Not thread safe: one host thread at a time per store.
 */
typedef struct flide_ckpt_store flide_ckpt_store;

/* *out (host) receives a store of n_slots slots numbered from first_slot.
 * Errors: FLIDE_E_INVALID_ARG (NULL out, first_slot < 0, n_slots < 1). */
flide_status flide_store_create(flide_ckpt_store** out, int32_t first_slot, int32_t n_slots);
/* Free the store (never touches device memory).  NULL is a no-op. */
void flide_store_destroy(flide_ckpt_store* store);
/* Longest committed checkpoint among the caller's n candidates (positions[i] >= 1, the digest of its
 * tokens 0..positions[i]-1 in digests[i]; host arrays).  On a hit *m_out / *slot_out receive the
 * position and slot and the slot's reference count grows by one (release it once the round that
 * resumes from it has completed); on a miss 0 and -1.  Errors: FLIDE_E_INVALID_ARG. */
flide_status flide_store_lookup(flide_ckpt_store* store, int32_t n, const int32_t* positions,
                                const uint64_t* digests, int32_t* m_out, int32_t* slot_out);
/* A slot for a new checkpoint of prefix (m, digest), to pass as a request's save_slot with save_m = m
 * (or as out_slot for the trunk's end, m = P).  The entry holds one reference and stays invisible to
 * lookups until flide_store_commit.  Errors: FLIDE_E_INVALID_ARG (m < 1, or the prefix is already
 * stored or reserved), FLIDE_E_CAPACITY (every slot is held by a round). */
flide_status flide_store_reserve(flide_ckpt_store* store, int32_t m, uint64_t digest, int32_t* slot_out);
/* Make a reserved slot visible to lookups: call it once the round that writes the checkpoint has
 * completed on the device.  Errors: FLIDE_E_INVALID_ARG (not a reserved slot of this store). */
flide_status flide_store_commit(flide_ckpt_store* store, int32_t slot);
/* Drop one reference of a slot returned by lookup or reserve.  A reservation released before its
 * commit frees the slot.  Errors: FLIDE_E_INVALID_ARG (not a held slot of this store). */
flide_status flide_store_release(flide_ckpt_store* store, int32_t slot);
/* stats (host, 7 entries): slots, used, committed, held, hits, misses, evictions. */
flide_status flide_store_stats(const flide_ckpt_store* store, int64_t* stats);

/* ------------------------------------------------------------------------
 * Context
 * ------------------------------------------------------------------------ */

/* Infrastructure (owner of the graph buckets of [KO] §어떻게 쓰나).
 * Create a context on HIP device `device` (makes it current on this thread);
 * *out (host) receives the library-owned handle, NULL on error.
 * Errors: FLIDE_E_INVALID_ARG (NULL out), FLIDE_E_HIP (no such device),
 * FLIDE_E_UNSUPPORTED (not gfx950). */
flide_status flide_create(flide_ctx** out, int32_t device);
/* Infrastructure.  Free graphs, pinned staging and rotary tables.  Never frees
 * caller memory.  Synchronises the device first.  NULL is a no-op. */
void flide_destroy(flide_ctx* ctx);
/* Infrastructure.  Message of the last failing call on this context ("" if
 * none; never NULL; owned by the context, valid until its next call). */
const char* flide_last_error(const flide_ctx* ctx);
/* Infrastructure.  The raw hipError_t of the last call on this context that
 * returned FLIDE_E_HIP (0 = hipSuccess if none did; 0 for a NULL context).
 * Calls that fail for other reasons leave it unchanged. */
int32_t flide_last_hip_error(const flide_ctx* ctx);

/* Per-round metadata write ([ZH] §方法步骤详情 third step: each round only
 * rewrites the device buffers of segment lengths, positions, key ranges and
 * state indices; [ZH] §方法步骤详情 first step: every row carries (j, c, t)).
 * Upload a metadata image and expand the per-row arrays on the device.
 * image (host): written by flide_plan_round for `caps`; dev_meta (device):
 * layout.dev_words int32 words.  The image is copied into library-owned pinned
 * staging before the call returns, so the caller may reuse `image` at once.
 * Errors: FLIDE_E_INVALID_ARG (NULL, header inconsistent with caps), FLIDE_E_HIP. */
flide_status flide_meta_upload(flide_ctx* ctx, const flide_caps* caps, const int32_t* image, int32_t* dev_meta,
                               void* stream);

/* ------------------------------------------------------------------------
 * Token-mixing kernels (every tensor is device memory owned by the caller)
 * ------------------------------------------------------------------------ */

/* Tree-masked varlen attention, full or sliding window ([ZH] §方法步骤详情:
 * key y is visible from query x iff j_y = j_x, c_y in {0, c_x}, t_y <= t_x, and
 * for a window layer t_x - t_y < W).  Rotary embedding at the metadata
 * positions (rotate-half pairs (i, i + d/2), angle t * theta^(-2i/d), fp64 host
 * table stored as fp32).  Grouped-query heads: q head h reads kv head
 * h / (Hq / Hkv).  Scores scaled by 1/sqrt(d); fp32 softmax and accumulation.
 *  Hq, Hkv, d   heads and head size; Hq % Hkv == 0; d a multiple of 8 in
 *               [8, 256] (bf16 with d == 128 or 256 runs on the MFMA path).
 *  window       0 = full attention, else W >= 1
 *  theta        rotary base
 *  max_pos      exclusive bound on every position of the rounds run (rotary table size)
 *  cache_rows, cache_slots  shape of the K/V cache (0 if no request resumes)
 *  deterministic accepted for symmetry with flide_gdn_params: attention always
 *               runs per-segment query tiles over position-aligned key tiles,
 *               so its bits never depend on the round's composition (no
 *               cheaper composition-dependent tiling exists here)             */
typedef struct {
  int32_t Hq, Hkv, d, window;
  double theta;
  int32_t max_pos;
  int32_t cache_rows;  /* rows per K/V cache slot (>= the largest m), 0 if no cache */
  int32_t cache_slots; /* slots of the K/V cache, 0 if no cache                     */
  int32_t dtype;       /* flide_dtype of q, k, v, caches and o                      */
  int32_t deterministic;
} flide_attn_params;

/* Infrastructure (sizes the scratch of the rotation of [ZH] §方法步骤详情).
 * Bytes of the workspace flide_fork_attn needs for `caps` (rotated keys and, on the
 * bf16 MFMA path, transposed values); *bytes (host) written on success.  Zero-fill the workspace once when allocating it:
 * columns between segments are read under a zero mask and must hold finite values. */
flide_status flide_attn_workspace_bytes(const flide_caps* caps, const flide_attn_params* p, int64_t* bytes);

/*  q        [T_cap, Hq, d]   queries, not yet rotated
 *  k, v     [T_cap, Hkv, d]  keys (not yet rotated) and values
 *  k_cache  [slots, cache_rows, Hkv, d] keys of positions 0..m-1, already
 *           rotated.  v_cache [slots, Hkv, d, cache_rows]: the matching values,
 *           stored transposed (position fastest) so value tiles load as rows.
 *           cache_rows must be a multiple of 8.  Read for requests with m > 0
 *           from slot ckpt_slot; may be NULL when no request resumes.
 *  o        [T_cap, Hq, d]   output rows 0..T-1 (tail rows untouched)
 *  workspace device scratch of flide_attn_workspace_bytes bytes
 * Errors: FLIDE_E_INVALID_ARG, FLIDE_E_UNSUPPORTED (dims/dtype), FLIDE_E_HIP. */
flide_status flide_fork_attn(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta,
                             const flide_attn_params* p, const void* q, const void* k, const void* v,
                             const void* k_cache, const void* v_cache, void* o, void* workspace, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving loops or
 * harnesses that forbid hipMalloc): flide_fork_attn without the workspace argument.  The rotated keys
 * and transposed values go to a device array of this library, one per GPU, that holds 64 MiB of
 * workspace (flide_attn_workspace_bytes(caps, p) must not exceed it: about 16k stream rows at 4 kv
 * heads of 256) plus a 16 MiB rotary-table region (max_pos * d * 4 bytes), used when the context
 * holds no table for (theta, d, max_pos) yet; writing that region the first time waits for `stream`.
 * The array is set up by flide_create and kept until the process ends.  Every call on one GPU shares
 * it and it keeps the last call's contents: calls that overlap on one GPU (other streams, other
 * threads, other contexts) race.  Nothing is allocated on the device.  Arguments and layouts as
 * flide_fork_attn; results are bit-identical to it.
 * Errors: FLIDE_E_CAPACITY (workspace or table above the array's size; nothing is launched), and as
 * flide_fork_attn. */
flide_status flide_fork_attn_noalloc(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta,
                                     const flide_attn_params* p, const void* q, const void* k, const void* v,
                                     const void* k_cache, const void* v_cache, void* o, void* stream);

/* Gated DeltaNet layer, two calls ([ZH] §前置知识 and §方法步骤详情; [KO]
 * §무엇과 다른가): causal depthwise conv over the raw q|k|v channels (width
 * conv_k, tap conv_k-1 multiplies the current row, no bias), optional SiLU,
 * per-head L2 normalisation of q and k (x / sqrt(sum x^2 + 1e-6)), then
 *     S_t = alpha_t S_{t-1} (I - eta_t k_t k_t^T) + eta_t v_t k_t^T,  o_t = S_t q_t
 * with an fp32 state S of [dv, dk] per head.
 *  phase 0 (FLIDE_GDN_TRUNKS): every trunk segment from a zero state and zero
 *     conv history, or, for m > 0, from state_pool/conv_pool[ckpt_slot]; writes
 *     S_P to state_pool[out_slot] and the last conv_k-1 raw trunk inputs to
 *     conv_pool[out_slot]; for save_m > 0 also the state after position
 *     save_m - 1 and the conv_k-1 raw inputs before save_m to save_slot.
 *  phase 1 (FLIDE_GDN_QUESTIONS): every question segment at once, each seeded
 *     by index from state_pool/conv_pool[its request's out_slot] (no copy);
 *     the pools are only read.
 * Parameters: H heads, dk = dv in {32, 64, 128} (bf16) or any <= 128 (f32),
 * conv_k in 1..4, act 0 = none, 1 = SiLU, chunk = rows per chunk (64).
 *  x          [T_cap, H*(2dk+dv)] raw inputs, channels q | k | v, head-major
 *  conv_w     [H*(2dk+dv), conv_k] fp32
 *  alpha, eta [T_cap, H] fp32
 *  state_pool [n_slots, H, dv, dk] fp32
 *  conv_pool  [n_slots, conv_k-1, H*(2dk+dv)] in the dtype of x
 *  o          [T_cap, H, dv] in the dtype of x (tail rows untouched)
 * Errors: FLIDE_E_INVALID_ARG, FLIDE_E_UNSUPPORTED, FLIDE_E_HIP.  A slot index
 * outside [0, n_slots) found on the device sets the device error word.
 * deterministic (the optional mode of [KO] §어떻게 쓰나, default on in the Python
 * binding): 1 = chunks of 64 rows from each segment's first row, so a request's
 * output bits do not depend on the rest of the round; 0 = chunk boundaries at
 * the multiples of 64 stream rows (and at an interior checkpoint), the grid of
 * a packed batch, under which a segment's bits depend on where it lands.  The
 * per-token kernel (f32, other head sizes) has no chunks and ignores it.     */
typedef enum { FLIDE_GDN_TRUNKS = 0, FLIDE_GDN_QUESTIONS = 1 } flide_gdn_phase;
typedef struct {
  int32_t H, dk, dv, conv_k;
  int32_t act;
  int32_t chunk;
  int32_t dtype;
  int32_t deterministic;
} flide_gdn_params;

/* The two halves of flide_fork_attn, for callers that schedule them apart;
 * flide_fork_attn is flide_attn_prepare followed by flide_attn_core on one stream.
 * flide_attn_prepare: rotary embedding of k at the metadata positions (the
 *   rotation of [ZH] §方法步骤详情) into `workspace`, and on the bf16 MFMA path the
 *   transposed copy of v (per segment, value columns starting 8-aligned).
 * flide_attn_core: the masked attention of q against the prepared workspace and
 *   the K/V cache.  v is read only on the f32 path (the MFMA path reads the
 *   transposed copy).  The workspace must hold what flide_attn_prepare wrote for
 *   the same metadata, params and k, v.
 * Arguments, layouts and errors as flide_fork_attn. */
flide_status flide_attn_prepare(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta,
                                const flide_attn_params* p, const void* k, const void* v, void* workspace,
                                void* stream);
flide_status flide_attn_core(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta,
                             const flide_attn_params* p, const void* q, const void* v, const void* k_cache,
                             const void* v_cache, void* o, const void* workspace, void* stream);

/* Interior checkpoint K/V ([KO] §어떻게 쓰나: a later round resumes at m from a
 * checkpoint holding the attention K/V of positions 0..m-1): for every request
 * of the metadata with save_m > 0, copy the rotated keys and the values of its
 * trunk positions 0..save_m-1 into k_cache/v_cache slot save_slot, in the cache
 * layouts of flide_fork_attn.  Positions below the request's resume point m come
 * from its ckpt_slot; the rest from `workspace` as flide_attn_prepare left it for
 * the same metadata (rotated keys; on the bf16 MFMA path the transposed values,
 * else the value rows of v).  Run it after flide_attn_prepare (or a whole round)
 * and before the workspace is reused.  p->cache_rows must be >= every save_m;
 * a slot or position outside the cache sets the device error word (read by
 * flide_check_device).  The GDN half of the checkpoint is written by
 * flide_fork_gdn phase 0.  Whole rounds (flide_graph_capture, flide_round_eager)
 * run this step themselves after each attention layer that has a K/V cache.
 * Errors: FLIDE_E_INVALID_ARG (NULL buffers, no cache), FLIDE_E_UNSUPPORTED, FLIDE_E_HIP. */
flide_status flide_attn_save_kv(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta,
                                const flide_attn_params* p, const void* v, const void* workspace, void* k_cache,
                                void* v_cache, void* stream);

flide_status flide_fork_gdn(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta,
                            const flide_gdn_params* p, int32_t phase, const void* x, const float* conv_w,
                            const float* alpha, const float* eta, float* state_pool, void* conv_pool,
                            int32_t n_slots, void* o, void* stream);

/* Selective readout, Eq. (1) ([KO] §어떻게 동작하나; [ZH] §方法步骤详情 fourth
 * step): for question i (stream order), h = H[qfin_row[i]] and
 * p_i(o) = softmax over o in O_i of w_o^T h, logits accumulated in fp32.
 *  h        [T_cap, hidden] (dtype)       w_opt [n_opt_rows, hidden] (dtype)
 *  opt_off  [n_qst + 1] int32 CSR offsets; opt_id [opt_off[n_qst]] rows of w_opt
 *  probs    [opt_off[n_qst]] fp32
 * Errors: FLIDE_E_INVALID_ARG, FLIDE_E_UNSUPPORTED, FLIDE_E_HIP; an option row
 * outside [0, n_opt_rows) found on the device sets the device error word.   */
typedef struct {
  int32_t hidden;
  int32_t dtype;
} flide_readout_params;

flide_status flide_readout(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta,
                           const flide_readout_params* p, const void* h, const void* w_opt,
                           const int32_t* opt_off, const int32_t* opt_id, int32_t n_opt_rows, float* probs,
                           void* stream);

/* ------------------------------------------------------------------------
 * Row-wise layers of a multi-layer hybrid stack
 * ------------------------------------------------------------------------
 * Every layer other than the token mixers acts on each row alone ([ZH]
 * §方法步骤详情 second step), so on the flat stream it runs over the rows
 * unchanged; after the last token mixer only the question-final rows are
 * needed ([ZH] §方法步骤详情 fourth step; [KO] §어떻게 쓰나, selective
 * readout).  Each call acts on a row set read from dev_meta at run time:
 * FLIDE_ROWS_ALL = stream rows [0, T), FLIDE_ROWS_QFINAL = the rows
 * qfin_row[0 .. n_qst); rows outside the set are left untouched, so one
 * captured graph serves every round of its capacity.  Tensors are row-major
 * over stream rows in the dtype given (f32 or bf16; gains, biases and gates
 * fp32); every pointer is caller-owned device memory.
 */
typedef enum { FLIDE_ROWS_ALL = 0, FLIDE_ROWS_QFINAL = 1 } flide_rows;

/* y[r] = x[r] / sqrt(mean(x[r]^2) + eps) * g   (x, y [T_cap, D]; g [D] fp32; fp32 accumulation).
 * x and y may be the same buffer.  Errors: FLIDE_E_INVALID_ARG, FLIDE_E_UNSUPPORTED, FLIDE_E_HIP. */
flide_status flide_rmsnorm(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta, int32_t rows,
                           int32_t dtype, int32_t D, const void* x, const float* g, float eps, void* y,
                           void* stream);
/* c[r, n] = sum_k a[r, k] w[n, k] (+ resid[r, n]) for n < N: a linear layer with its weight stored
 * [N, K] (out, in).  a has row stride lda >= K, c and resid row stride ldc >= N; resid may be NULL or c
 * itself (in-place residual add), never a.  fp32 accumulation (bf16: on MFMA, K a multiple of 32 and lda
 * of 8; f32: in order along K).  Errors: FLIDE_E_INVALID_ARG, FLIDE_E_UNSUPPORTED, FLIDE_E_HIP. */
flide_status flide_linear(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta, int32_t rows,
                          int32_t dtype, int32_t N, int32_t K, const void* a, int64_t lda, const void* w,
                          const void* resid, void* c, int64_t ldc, void* stream);
/* out[r, f] = silu(gu[r, f]) * gu[r, F + f]   (gu [T_cap, 2F]: gate | up; out [T_cap, F]).
 * Errors: FLIDE_E_INVALID_ARG, FLIDE_E_UNSUPPORTED, FLIDE_E_HIP. */
flide_status flide_swiglu(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta, int32_t rows,
                          int32_t dtype, int32_t F, const void* gu, void* out, void* stream);
/* The gates of a Gated DeltaNet layer from a projection z [T_cap, 2H] (dtype): alpha[r, h] =
 * sigmoid(z[r, h] + bias[h]), eta[r, h] = sigmoid(z[r, H + h] + bias[H + h]) (alpha, eta [T_cap, H] fp32,
 * the layout flide_fork_gdn reads), over all stream rows.  Errors: as flide_swiglu. */
flide_status flide_gdn_gates(flide_ctx* ctx, const flide_caps* caps, const int32_t* dev_meta, int32_t dtype,
                             int32_t H, const void* z, const float* bias, float* alpha, float* eta, void* stream);

/* ------------------------------------------------------------------------
 * Whole rounds: graph buckets per stream capacity ([ZH] §核心方法 and
 * §方法步骤详情 third step; [KO] §어떻게 쓰나)
 * ------------------------------------------------------------------------ */

/* Every buffer of one round at one capacity.  Layer 0 is a full-attention
 * layer; layer 1 (n_attn == 2) an optional sliding-window layer.  The GDN
 * layer runs phase 0 then phase 1; the readout runs last.  Buffers must stay
 * alive as long as a graph captured from them.                                */
typedef struct {
  flide_caps caps;
  int32_t* dev_meta;
  int32_t n_attn;
  flide_attn_params attn[2];
  const void* q[2];
  const void* k[2];
  const void* v[2];
  const void* k_cache[2];
  const void* v_cache[2];
  void* o_attn[2];
  void* attn_ws[2];
  flide_gdn_params gdn;
  const void* x;
  const float* conv_w;
  const float* alpha;
  const float* eta;
  float* state_pool;
  void* conv_pool;
  int32_t n_slots;
  void* o_gdn;
  flide_readout_params ro;
  const void* h;
  const void* w_opt;
  const int32_t* opt_off;
  const int32_t* opt_id;
  int32_t n_opt_rows;
  float* probs;
} flide_round_bufs;

/* Capture the whole round (metadata expansion, GDN phases 0 and 1, attention
 * layers, the checkpoint K/V of requests with save_m > 0 when the layer has a
 * K/V cache, readout) into HIP graphs (the four parts of
 * flide_graph_replay_parts) for capacity bufs->caps.  Launch shapes
 * depend only on the capacity; kernels read their work from the metadata.
 * *bucket_id receives the bucket's id.  Errors: FLIDE_E_INVALID_ARG,
 * FLIDE_E_UNSUPPORTED, FLIDE_E_HIP.                                           */
flide_status flide_graph_capture(flide_ctx* ctx, const flide_round_bufs* bufs, void* stream, int32_t* bucket_id);
/* Bucket choice ([KO] §어떻게 쓰나: the smallest captured graph that fits the
 * round).  Smallest live captured bucket whose capacity holds (T, R, n_q);
 * *bucket_id (host) written on success.  FLIDE_E_CAPACITY if none. */
flide_status flide_select_bucket(const flide_ctx* ctx, int32_t T, int32_t R, int32_t n_q, int32_t* bucket_id);
/* Graph replay ([ZH] §核心方法: rewrite the buffers, replay the same graph).
 * Upload `image` (host, planned for the bucket's caps) into the bucket's
 * metadata through double-buffered pinned staging, then launch the graph.
 * Errors: FLIDE_E_INVALID_ARG (no such or released bucket, NULL image),
 * FLIDE_E_CAPACITY (image planned for larger caps), FLIDE_E_HIP. */
flide_status flide_graph_replay(flide_ctx* ctx, int32_t bucket_id, const int32_t* image, void* stream);
/* Infrastructure (scheduling of the request-boundary sub-rounds of [KO]
 * §어떻게 쓰나).  The captured round in four parts: 0 metadata expansion,
 * 1 GDN call 1 (the trunks), 2 attention and checkpoint K/V, 3 GDN call 2
 * (the questions) and the readout.  flide_graph_replay_parts launches the
 * parts whose bit is set in `parts` (bit i = part i, 1 .. 15), in part order,
 * on `stream`; with bit 0 it first uploads `image` as flide_graph_replay does
 * (image is ignored otherwise).  All four in order is exactly
 * flide_graph_replay.  The caller orders parts 1 and 2 after part 0, part 3
 * after part 1 (the same stream, or events), and the next round's part 0 of
 * the bucket after every part of this one; parts 1 and 2 of one bucket may
 * run side by side, and so may parts of different buckets (different
 * buffers): a sub-round's trunk call alone fills only as many CUs as it has
 * (segment, head) pairs.  flide_graph_replay_front is parts 0 and 1 (the
 * front), flide_graph_replay_back parts 2 and 3 (the back).
 * Errors: FLIDE_E_INVALID_ARG (no such or released bucket, parts out of
 * range, NULL image with bit 0), FLIDE_E_CAPACITY (image planned for larger
 * caps), FLIDE_E_HIP.                                                        */
flide_status flide_graph_replay_parts(flide_ctx* ctx, int32_t bucket_id, const int32_t* image, int32_t parts,
                                      void* stream);
flide_status flide_graph_replay_front(flide_ctx* ctx, int32_t bucket_id, const int32_t* image, void* stream);
flide_status flide_graph_replay_back(flide_ctx* ctx, int32_t bucket_id, void* stream);
/* Infrastructure (the capacity buckets of [KO] §어떻게 쓰나 are captured at
 * init; a caller that frees a bucket's buffers releases its graph first).
 * Destroy bucket `bucket_id`'s graph and staging after the device is idle; the
 * id is never reused, and flide_graph_replay / flide_select_bucket skip it.
 * Errors: FLIDE_E_INVALID_ARG (no such or already released bucket), FLIDE_E_HIP. */
flide_status flide_graph_release(flide_ctx* ctx, int32_t bucket_id);
/* The same kernel sequence launched one by one (no graph), e.g. for a single
 * request above the largest capacity ([KO] §어떻게 쓰나).                      */
flide_status flide_round_eager(flide_ctx* ctx, const flide_round_bufs* bufs, const int32_t* image, void* stream);

/* Infrastructure (a measured ceiling beside the published bf16 MFMA peak; no
 * passage of the pages asks for it).  Runs a loop of independent bf16
 * 16x16x32 matrix products (eight accumulators per wave, 512 workgroups of
 * 256 threads, `iters` x 8 products per wave) on `stream` after one short
 * warm-up launch, synchronises the stream and writes the rate in TFLOP/s to
 * *tflops (host).  Allocates nothing on the device.
 * Errors: FLIDE_E_INVALID_ARG (iters < 1 or tflops NULL), FLIDE_E_HIP.      */
flide_status flide_measure_mfma_peak(int32_t iters, void* stream, double* tflops);

/* Infrastructure.  Synchronise `stream`, read and clear the device error word
 * of dev_meta (device).  Returns FLIDE_E_DEVICE (with a message) if a kernel
 * flagged bad metadata, FLIDE_E_HIP if the stream reports an error.          */
flide_status flide_check_device(flide_ctx* ctx, const flide_caps* caps, int32_t* dev_meta, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLIDE_H */
