// Host planner: flat-stream metadata of a round, the attention work list and the
// request-boundary split.  Pure host code (runs without a GPU).
//
// Stream order and per-row labels follow "Flide: Accelerating Decision Inference
// with Exact State Forking" §方法步骤详情 (trunks first in request order, then the
// question segments grouped by request; every row labelled (j, c, t), question
// positions continuing from P).  Splitting at request boundaries, tail-only
// padding and the eager path follow the Korean summary §어떻게 쓰나.
#include <algorithm>
#include <cstring>
#include <vector>

#include "flide_internal.hpp"

namespace flide {

flide_status compute_layout(const flide_caps& c, flide_meta_layout& L) {
  if (c.T_cap < 1 || c.R_cap < 1 || c.Q_cap < 0) return FLIDE_E_INVALID_ARG;
  if (c.T_cap > (1 << 28) || c.R_cap > (1 << 24) || c.Q_cap > (1 << 24)) return FLIDE_E_INVALID_ARG;
  std::memset(&L, 0, sizeof(L));
  L.seg_cap = c.R_cap + c.Q_cap;
  L.tile_rows = kTileRows;
  L.tile_cap = ((c.T_cap + kTileRows - 1) / kTileRows + L.seg_cap + kXcdClasses - 1) / kXcdClasses * kXcdClasses;
  int64_t o = 0;
  auto take = [&](int64_t n) {
    int64_t at = o;
    o = align_words(o + n);
    return at;
  };
  L.hdr = take(kHdrWords);
  L.seg_row0 = take(L.seg_cap);
  L.seg_len = take(L.seg_cap);
  L.seg_req = take(L.seg_cap);
  L.seg_branch = take(L.seg_cap);
  L.seg_pos0 = take(L.seg_cap);
  L.seg_state = take(L.seg_cap);
  L.seg_vcol0 = take(L.seg_cap);
  L.req_trunk_row0 = take(c.R_cap);
  L.req_P = take(c.R_cap);
  L.req_m = take(c.R_cap);
  L.req_ckpt = take(c.R_cap);
  L.req_out = take(c.R_cap);
  L.req_q_seg0 = take(c.R_cap);
  L.req_nq = take(c.R_cap);
  L.req_save_m = take(c.R_cap);
  L.req_save_slot = take(c.R_cap);
  L.qfin_row = take(c.Q_cap > 0 ? c.Q_cap : 1);
  L.tile_seg = take(int64_t(L.tile_cap) * kTileUnits);
  L.tile_row0 = take(int64_t(L.tile_cap) * kTileUnits);
  L.tile_swa = take(L.tile_cap);
  L.gdn_order = take(L.seg_cap);
  L.host_words = o;
  L.tok_j = take(c.T_cap);
  L.tok_c = take(c.T_cap);
  L.tok_t = take(c.T_cap);
  L.tile_desc = take(int64_t(L.tile_cap) * kTileDescWords);
  L.dev_error = take(4);
  L.dev_words = o;
  return FLIDE_OK;
}

static flide_status check_requests(const flide_request* reqs, int32_t R, int64_t* T, int64_t* n_qst) {
  if (R < 0 || (R > 0 && reqs == nullptr)) return FLIDE_E_INVALID_ARG;
  int64_t rows = 0, nq = 0;
  for (int32_t j = 0; j < R; ++j) {
    const flide_request& r = reqs[j];
    if (r.P < 0 || r.m < 0 || r.m > r.P || r.n_q < 0) return FLIDE_E_INVALID_ARG;
    if (r.n_q > 0 && r.q_len == nullptr) return FLIDE_E_INVALID_ARG;
    if (r.out_slot < 0) return FLIDE_E_INVALID_ARG;
    if (r.m > 0 && (r.ckpt_slot < 0 || r.ckpt_slot == r.out_slot)) return FLIDE_E_INVALID_ARG;
    // an interior checkpoint sits on a chunk boundary of the trunk (or at its end)
    if (r.save_m != 0 && (r.save_m <= r.m || r.save_m > r.P || r.save_slot < 0 ||
                          ((r.save_m - r.m) % kCheckpointChunk != 0 && r.save_m != r.P)))
      return FLIDE_E_INVALID_ARG;
    rows += r.P - r.m;
    for (int32_t i = 0; i < r.n_q; ++i) {
      if (r.q_len[i] < 1) return FLIDE_E_INVALID_ARG;
      rows += r.q_len[i];
    }
    nq += r.n_q;
    if (rows > (int64_t(1) << 30)) return FLIDE_E_INVALID_ARG;
  }
  // Slots written by the trunk call (outputs and new checkpoints) must be distinct from each other
  // and from every slot a resumed trunk reads, or two workgroups would race on a slot.
  std::vector<int32_t> outs, ckpts;
  for (int32_t j = 0; j < R; ++j) {
    outs.push_back(reqs[j].out_slot);
    if (reqs[j].save_m != 0) outs.push_back(reqs[j].save_slot);
    if (reqs[j].m > 0) ckpts.push_back(reqs[j].ckpt_slot);
  }
  std::sort(outs.begin(), outs.end());
  std::sort(ckpts.begin(), ckpts.end());
  if (std::adjacent_find(outs.begin(), outs.end()) != outs.end()) return FLIDE_E_INVALID_ARG;
  for (int32_t o : outs)
    if (std::binary_search(ckpts.begin(), ckpts.end(), o)) return FLIDE_E_INVALID_ARG;
  *T = rows;
  *n_qst = nq;
  return FLIDE_OK;
}

}  // namespace flide

using namespace flide;

extern "C" {

const char* flide_status_string(int32_t s) {
  switch (s) {
    case FLIDE_OK: return "ok";
    case FLIDE_E_INVALID_ARG: return "invalid argument";
    case FLIDE_E_CAPACITY: return "capacity exceeded";
    case FLIDE_E_UNSUPPORTED: return "unsupported shape or dtype";
    case FLIDE_E_HIP: return "HIP runtime error";
    case FLIDE_E_DEVICE: return "device-side metadata check failed";
    case FLIDE_E_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

const char* flide_version(void) { return "flide-mi355x 0.1 (gfx950)"; }

flide_status flide_meta_layout_for(const flide_caps* caps, flide_meta_layout* out) {
  if (!caps || !out) return FLIDE_E_INVALID_ARG;
  return compute_layout(*caps, *out);
}

flide_status flide_plan_sizes(const flide_request* reqs, int32_t R, int32_t* T, int32_t* n_seg, int32_t* n_qst) {
  int64_t t = 0, nq = 0;
  flide_status st = check_requests(reqs, R, &t, &nq);
  if (st != FLIDE_OK) return st;
  if (T) *T = int32_t(t);
  if (n_seg) *n_seg = int32_t(R + nq);
  if (n_qst) *n_qst = int32_t(nq);
  return FLIDE_OK;
}

flide_status flide_plan_round(const flide_request* reqs, int32_t R, const flide_caps* caps, int32_t* image,
                              int64_t image_words) {
  try {
    if (!caps || !image) return FLIDE_E_INVALID_ARG;
    flide_meta_layout L;
    flide_status st = compute_layout(*caps, L);
    if (st != FLIDE_OK) return st;
    if (image_words < L.host_words) return FLIDE_E_INVALID_ARG;
    int64_t T = 0, nq = 0;
    st = check_requests(reqs, R, &T, &nq);
    if (st != FLIDE_OK) return st;
    if (T > caps->T_cap || R > caps->R_cap || nq > caps->Q_cap) return FLIDE_E_CAPACITY;

    std::vector<int32_t> img(size_t(L.host_words), 0);
    int32_t* hdr = img.data() + L.hdr;
    int32_t* s_row0 = img.data() + L.seg_row0;
    int32_t* s_len = img.data() + L.seg_len;
    int32_t* s_req = img.data() + L.seg_req;
    int32_t* s_br = img.data() + L.seg_branch;
    int32_t* s_pos = img.data() + L.seg_pos0;
    int32_t* s_st = img.data() + L.seg_state;
    int32_t* r_row0 = img.data() + L.req_trunk_row0;
    int32_t* r_P = img.data() + L.req_P;
    int32_t* r_m = img.data() + L.req_m;
    int32_t* r_ck = img.data() + L.req_ckpt;
    int32_t* r_out = img.data() + L.req_out;
    int32_t* r_qs = img.data() + L.req_q_seg0;
    int32_t* r_nq = img.data() + L.req_nq;
    int32_t* r_sm = img.data() + L.req_save_m;
    int32_t* r_ss = img.data() + L.req_save_slot;
    int32_t* qfin = img.data() + L.qfin_row;
    int32_t* s_vc = img.data() + L.seg_vcol0;

    int32_t row = 0, seg = 0, max_pos = 0;
    // trunk segments: one per request, in request order (possibly empty)
    for (int32_t j = 0; j < R; ++j) {
      const flide_request& r = reqs[j];
      r_row0[j] = row;
      r_P[j] = r.P;
      r_m[j] = r.m;
      r_ck[j] = r.m > 0 ? r.ckpt_slot : -1;
      r_out[j] = r.out_slot;
      r_nq[j] = r.n_q;
      r_sm[j] = r.save_m;
      r_ss[j] = r.save_m != 0 ? r.save_slot : -1;
      s_row0[seg] = row;
      s_len[seg] = r.P - r.m;
      s_req[seg] = j;
      s_br[seg] = 0;
      s_pos[seg] = r.m;
      s_st[seg] = r.m > 0 ? r.ckpt_slot : -1;
      ++seg;
      row += r.P - r.m;
      max_pos = std::max(max_pos, r.P);
    }
    // question segments, grouped by request; positions continue from P
    int32_t qi = 0;
    for (int32_t j = 0; j < R; ++j) {
      const flide_request& r = reqs[j];
      r_qs[j] = seg;
      for (int32_t i = 0; i < r.n_q; ++i) {
        s_row0[seg] = row;
        s_len[seg] = r.q_len[i];
        s_req[seg] = j;
        s_br[seg] = i + 1;
        s_pos[seg] = r.P;
        s_st[seg] = r.out_slot;
        ++seg;
        row += r.q_len[i];
        qfin[qi++] = row - 1;
        max_pos = std::max(max_pos, r.P + r.q_len[i]);
      }
    }
    // Columns of the transposed value workspace: every segment starts at the first free column
    // congruent to its first position modulo 32, so a value tile aligned in position space (32
    // positions) is exactly one 32-column block of the tile-major workspace.
    {
      int64_t vend = 0;
      for (int32_t s = 0; s < seg; ++s) {
        const int64_t pos0 = s_pos[s];
        const int64_t vstart = vend + (((pos0 - vend) % 32) + 32) % 32;
        s_vc[s] = int32_t(vstart - pos0);
        vend = vstart + s_len[s];
      }
    }
    int32_t n_tiles = 0, tile_group = 0;
    // Attention work list, indexed by the kernel's tile position x.  A tile is kTileUnits units of
    // kUnitRows rows (unit u of position x: segment tile_seg[x kTileUnits + u], first row tile_row0[...],
    // segment -1 for none).  A trunk's tiles are kTileRows rows aligned to its start.  The questions of a
    // request are cut into units aligned to each question's start, and the request's question units are
    // packed four to a tile in question order, so a tile may hold rows of up to four sibling questions
    // (they share the request's cached and trunk keys; each sees its own rows only).  Cost = keys seen by
    // the tile's last row.  A request's tiles (trunk by
    // position, then its questions, which read the trunk's keys) are cut into contiguous groups of at
    // most about 1/16 of the round's cost; the groups go, heaviest first, to the least loaded of
    // kXcdClasses classes, and class c's tiles take positions c, c + 8, c + 16, ... group by group
    // (heaviest tile first within a group).  The kernel runs position x on XCD x mod 8, so a group's
    // key and value tiles are read into one L2, one or two groups at a time.  Unused positions hold
    // segment -1.  Tiles are independent, so the order does not change
    // any output bit.
    {
      constexpr int64_t kLongTileKeys = 4096;  // mean keys per tile above which the tile-group order is used
      constexpr int32_t kLongTileGroup = 64;   // positions per run: the workgroups of one XCD (32 CUs x 2)
      struct Tile {
        int64_t cost;
        int32_t seg[kTileUnits], row0[kTileUnits];
        int32_t pos;  // its position in the work list, once placed
      };
      std::vector<std::vector<Tile>> per_req(static_cast<size_t>(R));
      int64_t total = 0, n_all = 0;
      auto push = [&](Tile& t, std::vector<Tile>& out) {
        out.push_back(t);
        total += t.cost;
        ++n_all;
        t.cost = 0;
        for (int u = 0; u < kTileUnits; ++u) t.seg[u] = -1, t.row0[u] = 0;
      };
      Tile cur;
      cur.cost = 0, cur.pos = -1;
      for (int u = 0; u < kTileUnits; ++u) cur.seg[u] = -1, cur.row0[u] = 0;
      for (int32_t j = 0; j < R; ++j) {
        const flide_request& r = reqs[j];
        std::vector<Tile>& out = per_req[size_t(j)];
        for (int32_t a = 0; a < s_len[j]; a += kTileRows) {  // trunk: whole tiles of one segment
          for (int u = 0; u < kTileUnits && a + u * kUnitRows < s_len[j]; ++u)
            cur.seg[u] = j, cur.row0[u] = s_row0[j] + a + u * kUnitRows;
          cur.cost = int64_t(r.m) + std::min(a + kTileRows, s_len[j]);
          push(cur, out);
        }
        int nu = 0;  // question units: packed in question order
        for (int32_t i = 0; i < r.n_q; ++i) {
          const int32_t s = r_qs[j] + i;
          for (int32_t a = 0; a < s_len[s]; a += kUnitRows) {
            cur.seg[nu] = s, cur.row0[nu] = s_row0[s] + a;
            cur.cost = std::max(cur.cost, int64_t(r.P) + std::min(a + kUnitRows, s_len[s]));
            if (++nu == kTileUnits) {
              push(cur, out);
              nu = 0;
            }
          }
        }
        if (nu > 0) {
          push(cur, out);
          nu = 0;
        }
      }
      if (n_all > L.tile_cap) return FLIDE_E_INTERNAL;
      struct Group {
        int64_t cost;
        std::vector<Tile> tiles;
      };
      // Classes from request groups of at most 1/parts of the round's cost (heaviest group to the least
      // loaded class).
      std::vector<Tile> cls[kXcdClasses];
      auto make_classes = [&](int64_t parts) {
        const int64_t target = std::max<int64_t>(1, (total + parts - 1) / parts);
        std::vector<Group> groups;
        for (auto& rt : per_req) {
          Group cur{0, {}};
          for (const Tile& t : rt) {
            cur.tiles.push_back(t);
            cur.cost += t.cost;
            if (cur.cost >= target) {
              groups.push_back(std::move(cur));
              cur = Group{0, {}};
            }
          }
          if (!cur.tiles.empty()) groups.push_back(std::move(cur));
        }
        std::stable_sort(groups.begin(), groups.end(), [](const Group& x, const Group& y) { return x.cost > y.cost; });
        int64_t load[kXcdClasses] = {};
        for (auto& v : cls) v.clear();
        for (const Group& g : groups) {
          int c = 0;
          for (int k = 1; k < kXcdClasses; ++k)
            if (load[k] < load[c]) c = k;
          load[c] += g.cost;
          std::vector<Tile> gt = g.tiles;
          std::stable_sort(gt.begin(), gt.end(), [](const Tile& x, const Tile& y) { return x.cost > y.cost; });
          cls[c].insert(cls[c].end(), gt.begin(), gt.end());
        }
        size_t n = 0;
        for (auto& v : cls) n = std::max(n, v.size());
        return n;
      };
      // Groups of 1/32 of the cost balance the classes more finely: long-document full layer 7% faster than
      // with 1/16 (measured on MI355X).  Rounds whose tiles see thousands of keys each keep groups of 1/16:
      // the fan-out round's attention is 1% slower with 1/32, agent resume the same.  So do rounds whose
      // 1/32 classes do not fit the list.
      const bool long_tiles = total >= kLongTileKeys * n_all;
      if (long_tiles || make_classes(32) * kXcdClasses > size_t(L.tile_cap)) make_classes(16);
      size_t maxlen = 0;
      for (auto& v : cls) maxlen = std::max(maxlen, v.size());
      int32_t* t_seg = img.data() + L.tile_seg;
      int32_t* t_row = img.data() + L.tile_row0;
      int32_t* t_swa = img.data() + L.tile_swa;
      for (int32_t q = 0; q < L.tile_cap; ++q) t_swa[q] = -1;
      // Band order: the tiles heaviest first, cut into bands of kXcdClasses x kLongTileGroup tiles of
      // similar cost.  Within a band the tiles are ordered by request and dealt to the classes in runs of
      // up to kLongTileGroup, so each XCD takes a request-contiguous run of each band while every XCD gets
      // an equal share of every band.  emit(q, tile) places band position q (tile nullptr: unused); the
      // return value is the number of positions.
      auto band_order = [&](std::vector<Tile> all, auto&& emit) {
        std::stable_sort(all.begin(), all.end(), [](const Tile& x, const Tile& y) { return x.cost > y.cost; });
        const size_t band = size_t(kXcdClasses) * kLongTileGroup;
        size_t k0 = 0;  // first class index of the band
        for (size_t b0 = 0; b0 < all.size(); b0 += band) {
          const size_t nb = std::min(band, all.size() - b0);
          const size_t per = (nb + kXcdClasses - 1) / kXcdClasses;  // positions per class in this band
          std::stable_sort(all.begin() + b0, all.begin() + b0 + nb,
                           [&](const Tile& x, const Tile& y) { return s_req[x.seg[0]] < s_req[y.seg[0]]; });
          for (size_t k = 0; k < per * kXcdClasses; ++k)
            emit(int64_t((k0 + k % per) * kXcdClasses + k / per), k < nb ? &all[b0 + k] : nullptr);
          k0 += per;
        }
        return int64_t(k0) * kXcdClasses;
      };
      auto put = [&](int32_t x, const Tile* t) {  // position x of the work list (nullptr: unused)
        for (int u = 0; u < kTileUnits; ++u) {
          t_seg[int64_t(x) * kTileUnits + u] = t ? t->seg[u] : -1;
          t_row[int64_t(x) * kTileUnits + u] = t ? t->row0[u] : 0;
        }
      };
      if (int64_t(maxlen) * kXcdClasses <= L.tile_cap) {
        n_tiles = int32_t(maxlen) * kXcdClasses;
        // Rounds whose tiles see thousands of keys each stream long key ranges through L2: there the
        // kernel runs a class's positions in runs of kLongTileGroup per head group, so that the
        // workgroups resident on an XCD share one kv head's keys (measured on MI355X: 4-11% faster
        // attention on the fan-out and agent-resume rounds, 5% slower on short rounds).
        if (total >= kLongTileKeys * n_all) tile_group = kLongTileGroup;
        for (int32_t x = 0; x < n_tiles; ++x) put(x, nullptr);
        std::vector<Tile> all;
        for (int c = 0; c < kXcdClasses; ++c)
          for (size_t k = 0; k < cls[c].size(); ++k) {
            cls[c][k].pos = int32_t(k * kXcdClasses + size_t(c));
            put(cls[c][k].pos, &cls[c][k]);
            all.push_back(cls[c][k]);
          }
        // The classes balance the cost of full attention.  A windowed layer's tiles see at most W + 31
        // keys each, so its workgroups take the same tiles in band order (long-document window layer
        // 16% faster than in the classes' order, measured on MI355X); where the band order needs more
        // positions than the list holds, they take the positions in list order.
        std::vector<int32_t> swa(size_t(L.tile_cap), -1);
        const int64_t n_swa = band_order(all, [&](int64_t q, const Tile* t) {
          if (q < L.tile_cap) swa[size_t(q)] = t ? t->pos : -1;
        });
        for (int32_t q = 0; q < L.tile_cap; ++q)
          t_swa[q] = n_swa <= L.tile_cap ? swa[size_t(q)] : (q < n_tiles && t_seg[int64_t(q) * kTileUnits] >= 0 ? q : -1);
      } else {
        // Unbalanced classes (a few large requests): the band order for both layers.  With the tile-group
        // order the workgroups resident on an XCD then read one request's keys for one kv head (fan-out
        // round, measured on MI355X).
        std::vector<Tile> all;
        for (auto& v : cls) all.insert(all.end(), v.begin(), v.end());
        const int64_t n_band = band_order(all, [&](int64_t q, const Tile* t) {
          if (q < L.tile_cap) {
            put(int32_t(q), t);
            t_swa[q] = t ? int32_t(q) : -1;
          }
        });
        if (n_band > L.tile_cap) return FLIDE_E_INTERNAL;
        n_tiles = int32_t(n_band);
        if (total >= kLongTileKeys * n_all) tile_group = kLongTileGroup;
      }
    }
    // GDN work list: trunk segments, then question segments, each longest first (ties in stream
    // order), so that the chains that take longest start first.  Segments are independent, so the
    // order does not change any output bit.
    {
      int32_t* ord = img.data() + L.gdn_order;
      for (int32_t s = 0; s < seg; ++s) ord[s] = s;
      auto longer = [&](int32_t x, int32_t y) { return s_len[x] > s_len[y]; };
      std::stable_sort(ord, ord + R, longer);
      std::stable_sort(ord + R, ord + seg, longer);
    }
    hdr[H_T] = row;
    hdr[H_R] = R;
    hdr[H_NSEG] = seg;
    hdr[H_NQST] = qi;
    hdr[H_NTILES] = n_tiles;
    hdr[H_MAXPOS] = max_pos;
    hdr[H_TGROUP] = tile_group;
    hdr[H_MAGIC] = kMagic;
    std::memcpy(image, img.data(), size_t(L.host_words) * sizeof(int32_t));
    return FLIDE_OK;
  } catch (...) {
    return FLIDE_E_INTERNAL;
  }
}

flide_status flide_split_round(const flide_request* reqs, int32_t R, int32_t T_max, int32_t* sub_first,
                               int32_t* n_sub, uint8_t* eager) {
  if (T_max < 1 || !sub_first || !n_sub || (R > 0 && !eager)) return FLIDE_E_INVALID_ARG;
  int64_t T = 0, nq = 0;
  flide_status st = check_requests(reqs, R, &T, &nq);
  if (st != FLIDE_OK) return st;
  int32_t n = 0;
  sub_first[0] = 0;
  int64_t cur_rows = 0;
  int32_t cur_n = 0;
  for (int32_t j = 0; j < R; ++j) {
    const flide_request& r = reqs[j];
    int64_t rows = r.P - r.m;
    for (int32_t i = 0; i < r.n_q; ++i) rows += r.q_len[i];
    if (rows > T_max) {
      if (cur_n) {
        eager[n] = 0;
        sub_first[++n] = j;
      }
      eager[n] = 1;
      sub_first[++n] = j + 1;
      cur_rows = 0;
      cur_n = 0;
      continue;
    }
    if (cur_n && cur_rows + rows > T_max) {
      eager[n] = 0;
      sub_first[++n] = j;
      cur_rows = 0;
      cur_n = 0;
    }
    cur_rows += rows;
    ++cur_n;
  }
  if (cur_n) {
    eager[n] = 0;
    sub_first[++n] = R;
  }
  *n_sub = n;
  return FLIDE_OK;
}

}  // extern "C"
