// Host-only driver of the planner and the checkpoint store, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_abi_cpu.py (plain g++, no GPU code).  It runs seeded random
// rounds (valid and invalid) through flide_plan_sizes / flide_plan_round / flide_split_round into images
// allocated to exactly the size the layout names, and random operation sequences through the store;
// any out-of-bounds access, overflow or leak aborts the run.  Exit status 0 and a summary line on
// success; a logic check that fails prints its case and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "flide.h"

namespace {

struct Lcg {  // 64-bit linear congruential generator (Knuth's MMIX constants)
  uint64_t s;
  explicit Lcg(uint64_t seed) : s(seed * 2654435761u + 1) {}
  uint32_t next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return uint32_t(s >> 33);
  }
  int range(int lo, int hi) { return lo + int(next() % uint32_t(hi - lo + 1)); }  // inclusive
};

int fail(const char* what, int seed) {
  std::printf("FAIL %s (seed %d)\n", what, seed);
  return 1;
}

int plan_cases(int n_cases, int* n_ok, int* n_rejected) {
  for (int seed = 0; seed < n_cases; ++seed) {
    Lcg g(uint64_t(seed) + 1);
    const int R = g.range(0, 24);
    std::vector<std::vector<int32_t>> qlens(R);
    std::vector<flide_request> reqs(R);
    const bool make_invalid = g.range(0, 9) == 0;
    for (int j = 0; j < R; ++j) {
      flide_request& r = reqs[j];
      r.P = g.range(0, 400);
      r.m = g.range(0, 3) == 0 ? g.range(0, r.P) : 0;
      const int nq = g.range(0, 6);
      for (int i = 0; i < nq; ++i) qlens[j].push_back(g.range(1, 70));
      r.n_q = nq;
      r.q_len = nq ? qlens[j].data() : nullptr;
      r.out_slot = j;
      r.ckpt_slot = r.m > 0 ? R + j : -1;
      r.save_m = 0;
      r.save_slot = -1;
      if (r.P - r.m > 64 && g.range(0, 4) == 0) {
        r.save_m = r.m + 64 * g.range(1, (r.P - r.m) / 64);
        r.save_slot = 2 * R + j;
      }
    }
    if (make_invalid && R > 0) {  // one broken field: each must be rejected without touching the image
      flide_request& r = reqs[g.range(0, R - 1)];
      switch (g.range(0, 4)) {
        case 0: r.m = r.P + 1; break;
        case 1: if (r.n_q > 0) qlens[&r - reqs.data()][0] = 0; else r.n_q = -1; break;
        case 2: r.P = -5; break;
        case 3: if (r.m > 0) r.ckpt_slot = -1; else r.out_slot = -2; break;
        default: r.save_m = r.P + 3; r.save_slot = 9999; break;
      }
    }
    int32_t T = -1, n_seg = -1, n_qst = -1;
    const flide_status st = flide_plan_sizes(reqs.data(), R, &T, &n_seg, &n_qst);
    if (st != FLIDE_OK) {
      if (!make_invalid) return fail("valid round rejected by flide_plan_sizes", seed);
      ++*n_rejected;
      continue;
    }
    // capacities: exact, generous, or one short (must be FLIDE_E_CAPACITY)
    const int kind = g.range(0, 2);
    flide_caps caps{T + (kind == 1 ? g.range(1, 300) : 0), R + (kind == 1 ? 3 : 0), n_qst + (kind == 1 ? 2 : 0)};
    if (kind == 2 && T > 1) caps.T_cap = T - 1;
    if (caps.T_cap < 1) caps.T_cap = 1;
    if (caps.R_cap < 1) caps.R_cap = 1;
    if (caps.Q_cap < 1) caps.Q_cap = 1;
    flide_meta_layout L;
    if (flide_meta_layout_for(&caps, &L) != FLIDE_OK) return fail("layout", seed);
    std::vector<int32_t> image(size_t(L.host_words), 0x5A5A5A5A);  // exactly host_words: ASan sees overruns
    const flide_status ps = flide_plan_round(reqs.data(), R, &caps, image.data(), L.host_words);
    if (ps == FLIDE_OK) {
      ++*n_ok;
      if (image[L.hdr + 0] != T || image[L.hdr + 1] != R) return fail("header T/R", seed);
    } else if (ps == FLIDE_E_CAPACITY || ps == FLIDE_E_INVALID_ARG) {
      ++*n_rejected;
      for (int64_t i = 0; i < L.host_words; ++i)
        if (image[size_t(i)] != 0x5A5A5A5A) return fail("image written on error", seed);
    } else {
      return fail("unexpected status from flide_plan_round", seed);
    }
    // split at a random T_max
    std::vector<int32_t> first(size_t(R) + 1, -1);
    std::vector<uint8_t> eager(size_t(R > 0 ? R : 1), 0);
    int32_t n_sub = -1;
    const flide_status ss = flide_split_round(reqs.data(), R, g.range(1, 2000), first.data(), &n_sub, eager.data());
    if (ss == FLIDE_OK && (n_sub < 0 || n_sub > R)) return fail("split count", seed);
  }
  // NULL and size errors
  int32_t T = 0;
  if (flide_plan_sizes(nullptr, 3, &T, nullptr, nullptr) == FLIDE_OK) return fail("NULL requests accepted", 0);
  flide_caps bad{0, 0, 0};
  flide_meta_layout L;
  if (flide_meta_layout_for(&bad, &L) == FLIDE_OK) return fail("zero capacity accepted", 0);
  if (flide_meta_layout_for(nullptr, &L) == FLIDE_OK) return fail("NULL caps accepted", 0);
  return 0;
}

int store_cases(int n_cases, int64_t* n_ops) {
  for (int seed = 0; seed < n_cases; ++seed) {
    Lcg g(uint64_t(seed) + 1000);
    const int first = g.range(0, 5), n = g.range(1, 9);
    flide_ckpt_store* s = nullptr;
    if (flide_store_create(&s, first, n) != FLIDE_OK || !s) return fail("store create", seed);
    std::vector<int32_t> held;
    for (int op = 0; op < 300; ++op, ++*n_ops) {
      const int kind = g.range(0, 3);
      if (kind == 0) {  // reserve and (usually) commit a new prefix
        int32_t slot = -1;
        const int32_t m = g.range(1, 8) * 64;
        const uint64_t dg = uint64_t(g.range(0, 5));
        const flide_status st = flide_store_reserve(s, m, dg, &slot);
        if (st == FLIDE_OK) {
          if (slot < first || slot >= first + n) return fail("reserved slot outside the range", seed);
          if (g.range(0, 3) != 0) flide_store_commit(s, slot);
          held.push_back(slot);
        }
      } else if (kind == 1) {  // lookup among a few candidates
        int32_t pos[4];
        uint64_t dg[4];
        for (int i = 0; i < 4; ++i) {
          pos[i] = g.range(1, 8) * 64;
          dg[i] = uint64_t(g.range(0, 5));
        }
        int32_t m_out = -1, slot = -1;
        const flide_status st = flide_store_lookup(s, 4, pos, dg, &m_out, &slot);
        if (st == FLIDE_OK && slot >= 0) {
          if (slot < first || slot >= first + n) return fail("looked-up slot outside the range", seed);
          held.push_back(slot);
        }
      } else if (kind == 2 && !held.empty()) {  // release a held slot
        const size_t k = size_t(g.range(0, int(held.size()) - 1));
        if (flide_store_release(s, held[k]) != FLIDE_OK) return fail("release of a held slot", seed);
        held.erase(held.begin() + long(k));
      } else {  // misuse: must be rejected, never crash
        flide_store_release(s, first + n + 3);
        flide_store_commit(s, first - 1);
        int32_t slot;
        flide_store_reserve(s, 0, 1, &slot);
        flide_store_lookup(s, -1, nullptr, nullptr, nullptr, nullptr);
      }
    }
    int64_t stats[7];
    if (flide_store_stats(s, stats) != FLIDE_OK) return fail("stats", seed);
    flide_store_destroy(s);
  }
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  const int n_cases = argc > 1 ? std::atoi(argv[1]) : 3000;
  int ok = 0, rejected = 0;
  if (plan_cases(n_cases, &ok, &rejected)) return 1;
  int64_t ops = 0;
  if (store_cases(n_cases / 10 + 1, &ops)) return 1;
  std::printf("sanitized host run: %d rounds planned, %d rejected, %lld store operations\n", ok, rejected,
              static_cast<long long>(ops));
  return 0;
}
