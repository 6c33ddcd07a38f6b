// Prefix-match checkpoint store (host only).
//
// A later round may resume a request at position m from a checkpoint only if its tokens match the
// checkpoint's up to m (Korean summary §어떻게 쓰나).  The library never sees tokens, so the caller
// names a prefix by a digest of its first m tokens; the store maps (m, digest) to the pool slot that
// holds the checkpoint (GDN state, conv window and attention K/V of positions 0..m-1) and manages the
// slots of one pool range: a lookup returns the longest stored prefix among the caller's candidates,
// new checkpoints get a free slot or evict the least recently used entry that no round holds, and an
// entry becomes visible to lookups only once the caller commits it (after the round that writes it
// has completed on the device).
#include <algorithm>
#include <cstdint>
#include <map>
#include <new>
#include <utility>
#include <vector>

#include "flide_internal.hpp"

struct flide_ckpt_store {
  struct Entry {
    int32_t m = 0;
    uint64_t digest = 0;
    int32_t refs = 0;        // rounds that read or write the slot
    bool used = false;       // the slot holds (or is reserved for) a checkpoint
    bool visible = false;    // committed: lookups may return it
    uint64_t last_use = 0;   // LRU clock
  };
  int32_t first_slot = 0;
  std::vector<Entry> slots;
  std::map<std::pair<int32_t, uint64_t>, int32_t> index;  // (m, digest) -> local slot of a visible entry
  uint64_t clock = 0;
  int64_t hits = 0, misses = 0, evictions = 0;
};

namespace {

bool local_slot(const flide_ckpt_store* s, int32_t slot, int32_t* out) {
  const int32_t k = slot - s->first_slot;
  if (k < 0 || k >= int32_t(s->slots.size())) return false;
  *out = k;
  return true;
}

}  // namespace

extern "C" {

flide_status flide_store_create(flide_ckpt_store** out, int32_t first_slot, int32_t n_slots) {
  if (!out) return FLIDE_E_INVALID_ARG;
  *out = nullptr;
  if (first_slot < 0 || n_slots < 1 || int64_t(first_slot) + n_slots > (int64_t(1) << 30)) return FLIDE_E_INVALID_ARG;
  flide_ckpt_store* s = new (std::nothrow) flide_ckpt_store();
  if (!s) return FLIDE_E_INTERNAL;
  try {
    s->first_slot = first_slot;
    s->slots.resize(size_t(n_slots));
  } catch (...) {
    delete s;
    return FLIDE_E_INTERNAL;
  }
  *out = s;
  return FLIDE_OK;
}

void flide_store_destroy(flide_ckpt_store* s) { delete s; }

flide_status flide_store_lookup(flide_ckpt_store* s, int32_t n, const int32_t* positions, const uint64_t* digests,
                                int32_t* m_out, int32_t* slot_out) {
  if (!s || !m_out || !slot_out || n < 0 || (n > 0 && (!positions || !digests))) return FLIDE_E_INVALID_ARG;
  try {
    int32_t best_m = 0, best = -1;
    for (int32_t i = 0; i < n; ++i) {
      if (positions[i] < 1) return FLIDE_E_INVALID_ARG;
      if (positions[i] <= best_m) continue;
      auto it = s->index.find({positions[i], digests[i]});
      if (it != s->index.end()) {
        best_m = positions[i];
        best = it->second;
      }
    }
    if (best < 0) {
      ++s->misses;
      *m_out = 0;
      *slot_out = -1;
      return FLIDE_OK;
    }
    auto& e = s->slots[size_t(best)];
    ++e.refs;
    e.last_use = ++s->clock;
    ++s->hits;
    *m_out = best_m;
    *slot_out = s->first_slot + best;
    return FLIDE_OK;
  } catch (...) {
    return FLIDE_E_INTERNAL;
  }
}

flide_status flide_store_reserve(flide_ckpt_store* s, int32_t m, uint64_t digest, int32_t* slot_out) {
  if (!s || !slot_out || m < 1) return FLIDE_E_INVALID_ARG;
  try {
    if (s->index.count({m, digest})) return FLIDE_E_INVALID_ARG;  // already stored: look it up instead
    for (const auto& e : s->slots)
      if (e.used && !e.visible && e.m == m && e.digest == digest) return FLIDE_E_INVALID_ARG;  // already reserved
    int32_t pick = -1;
    for (int32_t k = 0; k < int32_t(s->slots.size()); ++k)
      if (!s->slots[size_t(k)].used) {
        pick = k;
        break;
      }
    if (pick < 0) {  // evict the least recently used committed entry that no round holds
      for (int32_t k = 0; k < int32_t(s->slots.size()); ++k) {
        const auto& e = s->slots[size_t(k)];
        if (e.visible && e.refs == 0 && (pick < 0 || e.last_use < s->slots[size_t(pick)].last_use)) pick = k;
      }
      if (pick < 0) return FLIDE_E_CAPACITY;
      auto& v = s->slots[size_t(pick)];
      s->index.erase({v.m, v.digest});
      ++s->evictions;
    }
    auto& e = s->slots[size_t(pick)];
    e = flide_ckpt_store::Entry();
    e.m = m;
    e.digest = digest;
    e.refs = 1;
    e.used = true;
    e.visible = false;
    e.last_use = ++s->clock;
    *slot_out = s->first_slot + pick;
    return FLIDE_OK;
  } catch (...) {
    return FLIDE_E_INTERNAL;
  }
}

flide_status flide_store_commit(flide_ckpt_store* s, int32_t slot) {
  int32_t k = 0;
  if (!s || !local_slot(s, slot, &k)) return FLIDE_E_INVALID_ARG;
  auto& e = s->slots[size_t(k)];
  if (!e.used || e.visible) return FLIDE_E_INVALID_ARG;
  try {
    s->index[{e.m, e.digest}] = k;
  } catch (...) {
    return FLIDE_E_INTERNAL;
  }
  e.visible = true;
  return FLIDE_OK;
}

flide_status flide_store_release(flide_ckpt_store* s, int32_t slot) {
  int32_t k = 0;
  if (!s || !local_slot(s, slot, &k)) return FLIDE_E_INVALID_ARG;
  auto& e = s->slots[size_t(k)];
  if (!e.used || e.refs < 1) return FLIDE_E_INVALID_ARG;
  --e.refs;
  if (!e.visible && e.refs == 0) e = flide_ckpt_store::Entry();  // a reservation abandoned before its commit
  return FLIDE_OK;
}

flide_status flide_store_stats(const flide_ckpt_store* s, int64_t* stats) {
  if (!s || !stats) return FLIDE_E_INVALID_ARG;
  int64_t used = 0, visible = 0, pinned = 0;
  for (const auto& e : s->slots) {
    used += e.used;
    visible += e.visible;
    pinned += e.refs > 0;
  }
  stats[0] = int64_t(s->slots.size());
  stats[1] = used;
  stats[2] = visible;
  stats[3] = pinned;
  stats[4] = s->hits;
  stats[5] = s->misses;
  stats[6] = s->evictions;
  return FLIDE_OK;
}

}  // extern "C"
