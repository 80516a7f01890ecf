// Host-side driver for the sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer on the
// host code only): the pager under a long random sequence of reserve / commit / evict / restore /
// resident / table calls with its invariants checked after every step, and every entry point's
// argument checks, which return before any HIP call (so no GPU is needed).  Exit status 0 when
// every check holds; the sanitizers abort on the first memory or undefined-behaviour error.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "ring_kv.h"

static int failures = 0;
#define CHECK(c)                                                       \
  do {                                                                 \
    if (!(c)) {                                                        \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

// Every slot is either free or held by exactly one table entry; paged-out entries sit below the
// committed whole chunks; the resident list is the table's entries with a slot, in order.
static void check_pager(const rkv_pager* p, int32_t n_slots, int32_t n_table) {
  std::vector<int32_t> tab(n_table);
  CHECK(rkv_pager_table(p, tab.data(), n_table) == RKV_OK);
  const int64_t ctx = rkv_pager_ctx_len(p);
  std::set<int32_t> held;
  int32_t with_slot = 0;
  for (int32_t c = 0; c < n_table; ++c) {
    if (tab[c] >= 0) {
      CHECK(tab[c] < n_slots);
      CHECK(held.insert(tab[c]).second);
      ++with_slot;
    } else if (tab[c] == RKV_PAGED_OUT) {
      CHECK(c < ctx / RKV_CHUNK);
    } else {
      CHECK(tab[c] == -1);
    }
  }
  CHECK(rkv_pager_free_slots(p) + with_slot == n_slots);
  const int32_t k = rkv_pager_resident(p, nullptr, nullptr, 0);
  CHECK(k == with_slot);
  std::vector<int32_t> ids(k > 0 ? k : 1), slots(k > 0 ? k : 1);
  CHECK(rkv_pager_resident(p, ids.data(), slots.data(), k) == k);
  for (int32_t i = 0; i < k; ++i) {
    CHECK(tab[ids[i]] == slots[i]);
    if (i > 0) CHECK(ids[i] > ids[i - 1]);
  }
}

static void pager_random(uint32_t seed) {
  std::mt19937 g(seed);
  const int32_t n_slots = 48, n_table = 400;
  rkv_pager* p = rkv_pager_create(n_slots, n_table);
  CHECK(p != nullptr);
  int32_t slots[RKV_MAX_APPEND_CHUNKS];
  for (int step = 0; step < 3000; ++step) {
    const int op = (int)(g() % 4);
    const int64_t ctx = rkv_pager_ctx_len(p);
    if (op <= 1) {                                      // a block: reserve then commit
      const int32_t n = 1 + (int32_t)(g() % (op == 0 ? 16 : 300));
      int32_t first = -1, n_new = -1;
      const int32_t st = rkv_pager_reserve(p, n, &first, &n_new, slots);
      if (st == RKV_OK) {
        CHECK(first == (int32_t)((ctx + RKV_CHUNK - 1) / RKV_CHUNK));
        CHECK(n_new >= 0 && n_new <= RKV_MAX_APPEND_CHUNKS);
        CHECK(rkv_pager_reserve(p, 1, &first, &n_new, slots) == RKV_ERR_ARG);   // one pending
        check_pager(p, n_slots, n_table);
        CHECK(rkv_pager_commit(p, (int32_t)(g() % (n + 1))) == RKV_OK);
      } else {
        CHECK(st == RKV_ERR_TABLE);
        if (ctx / RKV_CHUNK > 100) {                     // start over when the table fills
          rkv_pager_destroy(p);
          p = rkv_pager_create(n_slots, n_table);
        }
      }
    } else if (op == 2) {                               // evict some whole committed chunks
      std::vector<int32_t> tab(n_table);
      rkv_pager_table(p, tab.data(), n_table);
      std::vector<int32_t> cand;
      for (int32_t c = 0; c < ctx / RKV_CHUNK; ++c)
        if (tab[c] >= 0) cand.push_back(c);
      std::shuffle(cand.begin(), cand.end(), g);
      cand.resize(std::min<size_t>(cand.size(), g() % 6));
      std::vector<int32_t> out(cand.size() + 1);
      CHECK(rkv_pager_evict(p, cand.data(), (int32_t)cand.size(), out.data()) == RKV_OK);
      if (!cand.empty()) {                              // the same chunk again: rejected
        int32_t again = cand[0];
        CHECK(rkv_pager_evict(p, &again, 1, out.data()) == RKV_ERR_ARG);
      }
    } else {                                            // restore some paged-out chunks
      std::vector<int32_t> tab(n_table);
      rkv_pager_table(p, tab.data(), n_table);
      std::vector<int32_t> cand;
      for (int32_t c = 0; c < n_table; ++c)
        if (tab[c] == RKV_PAGED_OUT) cand.push_back(c);
      std::shuffle(cand.begin(), cand.end(), g);
      cand.resize(std::min<size_t>(cand.size(), g() % 6));
      std::vector<int32_t> out(cand.size() + 1);
      const int32_t st = rkv_pager_restore(p, cand.data(), (int32_t)cand.size(), out.data());
      CHECK(st == RKV_OK || (st == RKV_ERR_TABLE && (int32_t)cand.size() > rkv_pager_free_slots(p)));
    }
    check_pager(p, n_slots, n_table);
  }
  rkv_pager_destroy(p);
}

static void argument_checks() {
  alignas(16) char dummy[64];
  void* P = dummy;
  rkv_attn_dims d{16, 16, 4, 128, 0.f, RKV_BF16};
  rkv_attn_dims bad = d;
  bad.n_q_heads = 15;                                   // not a multiple of n_kv_heads
  float* out = reinterpret_cast<float*>(dummy);
  int32_t pt[4] = {0, 1, 2, 3};
  CHECK(verify_attn_paged(&bad, P, P, P, pt, 4, 4, 64, 256, 0, P, 1 << 20, out, nullptr, nullptr) < 0);
  CHECK(verify_attn_paged(&d, nullptr, P, P, pt, 4, 4, 64, 256, 0, P, 1 << 20, out, nullptr, nullptr) == RKV_ERR_NULL);
  CHECK(verify_attn_paged(&d, P, P, P, pt, 3, 4, 64, 256, 0, P, 1 << 20, out, nullptr, nullptr) == RKV_ERR_TABLE);
  CHECK(verify_attn_paged(&d, P, P, P, pt, 4, 4, 32, 256, 0, P, 1 << 20, out, nullptr, nullptr) == RKV_ERR_TABLE);
  CHECK(verify_attn_paged(&d, P, P, P, pt, 4, 4, 64, 8, 0, P, 1 << 20, out, nullptr, nullptr) == RKV_ERR_SHAPE);
  CHECK(verify_attn_paged(&d, P, P, P, pt, 4, 4, 64, 256, 0, nullptr, 0, out, nullptr, nullptr) == RKV_ERR_WORKSPACE);
  CHECK(verify_attn_paged_workspace_bytes(&bad, 256, 64, 0) == 0);
  CHECK(verify_attn_ring(&d, P, P, P, 30000, 1, 2048, 512, 0, P, 1 << 20, out, nullptr, nullptr) == RKV_ERR_RING);
  CHECK(verify_attn_ring(&d, P, P, P, 30000, 30000 % 2048, 520, 512, 0, P, 1 << 20, out, nullptr, nullptr) == RKV_ERR_RING);
  CHECK(decode_attn_ref_layout(&d, P, P, P, 8, 0, 0, P, 1 << 20, out, nullptr, nullptr) == RKV_ERR_SHAPE);
  int32_t prop[16] = {0};
  int32_t acc = 0, com[17];
  CHECK(verify_accept(out, 16, 0, prop, &acc, com, nullptr, P, 1 << 20, nullptr) == RKV_ERR_SHAPE);
  CHECK(verify_accept(out, 256, 10, prop, &acc, com, nullptr, P, 1 << 20, nullptr) == RKV_ERR_SHAPE);
  CHECK(verify_accept(out, 16, 1000, prop, &acc, com, nullptr, nullptr, 0, nullptr) == RKV_ERR_WORKSPACE);
  const int32_t ids_rep[2] = {5, 5}, slots_ok[2] = {0, 1};
  CHECK(kv_page_out(P, P, 4, 128, 4, slots_ok, ids_rep, 2, P, P, 10, P, 1 << 30, nullptr) == RKV_ERR_ARG);
  const int32_t ids_far[1] = {10}, slot_bad[1] = {7};
  CHECK(kv_page_out(P, P, 4, 128, 4, slots_ok, ids_far, 1, P, P, 10, P, 1 << 30, nullptr) == RKV_ERR_ARG);
  CHECK(kv_page_in(P, P, 10, ids_rep, slot_bad, 1, P, P, 4, 128, 4, P, 1 << 30, nullptr) == RKV_ERR_TABLE);
  CHECK(kv_page_in(P, P, 10, ids_rep, slots_ok, 1, P, P, 4, 100, 4, P, 1 << 30, nullptr) == RKV_ERR_SHAPE);
  const int32_t res_ids[3] = {0, 2, 1};                 // not increasing
  CHECK(verify_attn_paged_resident(&d, P, P, P, pt, res_ids, 3, 4, 200, 0, P, 1 << 20, out, nullptr, nullptr) == RKV_ERR_TABLE);
  const int32_t res_tail[2] = {0, 1};                   // the block's chunk 3 is not listed
  CHECK(verify_attn_paged_resident(&d, P, P, P, pt, res_tail, 2, 4, 256, 0, P, 1 << 20, out, nullptr, nullptr) == RKV_ERR_TABLE);
  int32_t first = 0, n_new = 0, sl[RKV_MAX_APPEND_CHUNKS];
  CHECK(rkv_pager_reserve(nullptr, 4, &first, &n_new, sl) == RKV_ERR_NULL);
  CHECK(rkv_pager_create(0, 4) == nullptr);
  for (int32_t s = -9; s <= 0; ++s) CHECK(rkv_status_str(s) != nullptr);
}

int main() {
  argument_checks();
  for (uint32_t seed = 1; seed <= 4; ++seed) pager_random(seed);
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("sanitized host checks passed\n");
  return 0;
}
