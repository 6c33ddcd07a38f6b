// Internal declarations shared by the host planner, the C ABI and the kernels.
#pragma once

#include <stdint.h>

#include "../../include/flide.h"

namespace flide {

// Query rows per attention work tile: kTileUnits units of kUnitRows rows.  A unit holds rows of one segment;
// a tile's units are consecutive rows of one trunk, or rows of up to four sibling questions.
constexpr int kTileRows = 32;
constexpr int kUnitRows = 8;
constexpr int kTileUnits = kTileRows / kUnitRows;
// XCDs of the chip: workgroup i of a grid runs on XCD i mod kXcdClasses.
constexpr int kXcdClasses = 8;
// int32 words of one attention work-list descriptor (filled on the device by meta_expand).
constexpr int kTileDescWords = 48;
// rows per GDN chunk: an interior checkpoint of a trunk sits at a multiple of it from the resume point
constexpr int kCheckpointChunk = 64;
// Descriptor words: the tile (segment of unit 0, -1 for an unused position; question flag; the request's
// P, m, checkpoint slot, trunk row and value-column offsets; the first and last query position over its
// units; the number of own-key ranges), then per unit u at TD_UNIT + 4 u: first row, rows (0: no unit),
// first position, own range; per own range k at TD_OWN + 4 k: row offset, value-column offset, first and
// one-past-last position.  An own range is one segment's rows (a trunk, or one question).
enum TileDesc { TD_SEG, TD_QUESTION, TD_P, TD_M, TD_CKPT, TD_ROFF_TRUNK, TD_VOFF_TRUNK, TD_QPOS_MIN, TD_QPOS_MAX,
                TD_NOWN, TD_UNIT = 16, TD_OWN = 32 };
enum TileUnit { TU_ROW0, TU_NROWS, TU_QPOS0, TU_OWN };
enum TileOwn { TO_ROFF, TO_VOFF, TO_LO, TO_HI };
// Words of the metadata header.
constexpr int kHdrWords = 64;
constexpr int32_t kMagic = 0x464C4944;  // 'FLID'

// Device scratch of the allocation-free attention entry point (one array per GPU, in noalloc.hip).
constexpr int64_t kNoAllocWorkspaceBytes = int64_t(64) << 20;  // attention workspace
constexpr int64_t kNoAllocTableBytes = int64_t(16) << 20;      // rotary table: max_pos * d * 4 bytes
// Takes the array's device address on `device` (current) once and clears it; hipError_t as int.
int noalloc_scratch_init(int device);
void* noalloc_workspace(int device);
float* noalloc_table(int device, double theta, int d, int max_pos, bool* holds, bool claim);

// Header fields.
enum : int {
  H_T = 0,
  H_R = 1,
  H_NSEG = 2,
  H_NQST = 3,
  H_NTILES = 4,
  H_MAXPOS = 5,
  H_TGROUP = 6,  // attention work order: 0 = head groups of a position together, n > 0 = runs of n positions
  H_MAGIC = 15,
};

// Device error bits.
enum : int32_t {
  E_HEADER = 1,     // header inconsistent with the capacity
  E_POSITION = 2,   // a position outside the rotary table
  E_SLOT = 4,       // a state slot outside the pool
  E_OPTION = 8,     // an option row outside w_opt
  E_CACHE = 16,     // a resume position beyond the K/V cache rows
  E_SEGMENT = 32,   // a segment/tile entry outside the stream
};

inline int64_t align_words(int64_t x) { return (x + 63) & ~int64_t(63); }

// Offsets of a metadata image (see flide_meta_layout in flide.h).
flide_status compute_layout(const flide_caps& caps, flide_meta_layout& L);

// Device pointers into one metadata image, passed by value to kernels.
struct MetaView {
  const int32_t* hdr;
  const int32_t* seg_row0;
  const int32_t* seg_len;
  const int32_t* seg_req;
  const int32_t* seg_branch;
  const int32_t* seg_pos0;
  const int32_t* seg_state;
  const int32_t* seg_vcol0;
  const int32_t* req_trunk_row0;
  const int32_t* req_P;
  const int32_t* req_m;
  const int32_t* req_ckpt;
  const int32_t* req_out;
  const int32_t* req_q_seg0;
  const int32_t* req_nq;
  const int32_t* req_save_m;
  const int32_t* req_save_slot;
  const int32_t* qfin_row;
  const int32_t* tile_seg;
  const int32_t* tile_row0;
  const int32_t* tile_swa;
  const int32_t* gdn_order;
  int32_t* tok_j;
  int32_t* tok_c;
  int32_t* tok_t;
  int32_t* tile_desc;
  int32_t* dev_error;
  int32_t T_cap, R_cap, Q_cap, seg_cap, tile_cap;
};

inline MetaView make_view(int32_t* base, const flide_meta_layout& L, const flide_caps& c) {
  MetaView v;
  v.hdr = base + L.hdr;
  v.seg_row0 = base + L.seg_row0;
  v.seg_len = base + L.seg_len;
  v.seg_req = base + L.seg_req;
  v.seg_branch = base + L.seg_branch;
  v.seg_pos0 = base + L.seg_pos0;
  v.seg_state = base + L.seg_state;
  v.seg_vcol0 = base + L.seg_vcol0;
  v.req_trunk_row0 = base + L.req_trunk_row0;
  v.req_P = base + L.req_P;
  v.req_m = base + L.req_m;
  v.req_ckpt = base + L.req_ckpt;
  v.req_out = base + L.req_out;
  v.req_q_seg0 = base + L.req_q_seg0;
  v.req_nq = base + L.req_nq;
  v.req_save_m = base + L.req_save_m;
  v.req_save_slot = base + L.req_save_slot;
  v.qfin_row = base + L.qfin_row;
  v.tile_seg = base + L.tile_seg;
  v.tile_row0 = base + L.tile_row0;
  v.tile_swa = base + L.tile_swa;
  v.gdn_order = base + L.gdn_order;
  v.tok_j = base + L.tok_j;
  v.tok_c = base + L.tok_c;
  v.tok_t = base + L.tok_t;
  v.tile_desc = base + L.tile_desc;
  v.dev_error = base + L.dev_error;
  v.T_cap = c.T_cap;
  v.R_cap = c.R_cap;
  v.Q_cap = c.Q_cap;
  v.seg_cap = L.seg_cap;
  v.tile_cap = L.tile_cap;
  return v;
}

// ---- kernel launchers (defined in the .hip files); all return a hipError_t as int ----
int launch_meta_expand(const MetaView& mv, void* stream);
int launch_clear_error(const MetaView& mv, void* stream);

struct RopeArgs {
  const float* table;  // [max_pos, d/2, 2]: (cos, sin) of every position and pair
  int32_t max_pos;
};

int launch_rope_k(const MetaView& mv, const flide_attn_params& p, const RopeArgs& rope, const void* k,
                  void* k_rot, void* stream);
// Rotates keys (and, on the MFMA path, transposes values) into `workspace`.
int launch_attn_prepare(const MetaView& mv, const flide_attn_params& p, const RopeArgs& rope, const void* k,
                        const void* v, void* workspace, void* stream);
// The masked attention over a prepared workspace (the f32 path reads values from v).
int launch_attn_core(const MetaView& mv, const flide_attn_params& p, const RopeArgs& rope, const void* q,
                     const void* v, const void* k_cache, const void* v_cache, void* o, const void* workspace,
                     void* stream);
// Interior checkpoints: K/V of positions 0..save_m-1 of every saving request into its cache slot.
int launch_attn_save_kv(const MetaView& mv, const flide_attn_params& p, const void* v, const void* workspace,
                        void* k_cache, void* v_cache, void* stream);
// Row-wise layers of a stack (stack_kernels.hip); rows_mode 0 = stream rows [0, T), 1 = question-final rows.
int launch_rmsnorm(const MetaView& mv, int rows_mode, int dtype, int D, const void* x, const float* g, float eps,
                   void* y, void* stream);
int launch_swiglu(const MetaView& mv, int rows_mode, int dtype, int F, const void* gu, void* out, void* stream);
int launch_gates(const MetaView& mv, int dtype, int H, const void* z, const float* bias, float* alpha, float* eta,
                 void* stream);
int launch_linear(const MetaView& mv, int rows_mode, int dtype, int N, int K, const void* a, int64_t lda,
                  const void* w, const void* resid, void* c, int64_t ldc, void* stream);
bool attn_uses_mfma(const flide_attn_params& p);
int64_t attn_workspace_bytes(const flide_caps& c, const flide_attn_params& p);
int launch_gdn(const MetaView& mv, const flide_gdn_params& p, int phase, const void* x, const float* conv_w,
               const float* alpha, const float* eta, float* state_pool, void* conv_pool, int32_t n_slots,
               void* o, void* stream);
int launch_readout(const MetaView& mv, const flide_readout_params& p, const void* h, const void* w_opt,
                   const int32_t* opt_off, const int32_t* opt_id, int32_t n_opt_rows, float* probs,
                   void* stream);

}  // namespace flide
