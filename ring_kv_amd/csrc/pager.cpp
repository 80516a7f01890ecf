// Host-side pager of the paged KV pool: the free list of pool slots and a host copy of the
// page table for one sequence (lucebox post "Laguna XS 2.1 33B on a RTX 3090: 296 tok/s peak,
// 152 tok/s at 256K context", "Three optimizations", item 1: the full-attention layers keep
// 64-token chunks in a pool located through a page table).  A verify block first reserves the
// chunks its rows start, and after the accept commits the rows it keeps; chunks that end up
// holding no committed position return to the free list.  Whole committed chunks can be paged
// out to host memory (their slots return to the free list) and back in (same post, same item:
// chunks move between the pool and host memory).
#include "ring_kv.h"

#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

struct rkv_pager {
  int32_t n_slots;
  std::vector<int32_t> table;     // logical chunk -> slot, -1 for none, RKV_PAGED_OUT on the host
  std::vector<int32_t> free;      // stack: back() is handed out next
  int64_t ctx = 0;                // committed positions
  // the pending block (between reserve and commit)
  bool pending = false;
  int32_t pend_n = 0;
  int32_t pend_first = 0;         // first chunk the block started
  int32_t pend_new = 0;           // chunks it started
};

namespace {

constexpr int64_t kChunk = RKV_CHUNK;

int64_t ceil_chunks(int64_t positions) { return (positions + kChunk - 1) / kChunk; }

}  // namespace

extern "C" {

rkv_pager* rkv_pager_create(int32_t n_slots, int32_t n_table) {
  if (n_slots < 1 || n_table < 1) return nullptr;
  rkv_pager* p = new (std::nothrow) rkv_pager;
  if (p == nullptr) return nullptr;
  p->n_slots = n_slots;
  p->table.assign((size_t)n_table, -1);
  p->free.reserve((size_t)n_slots);
  for (int32_t s = n_slots - 1; s >= 0; --s) p->free.push_back(s);   // hands out 0, 1, 2, ...
  return p;
}

void rkv_pager_destroy(rkv_pager* p) { delete p; }

int64_t rkv_pager_ctx_len(const rkv_pager* p) { return p == nullptr ? -1 : p->ctx; }

int32_t rkv_pager_free_slots(const rkv_pager* p) {
  return p == nullptr ? -1 : (int32_t)p->free.size();
}

int32_t rkv_pager_table(const rkv_pager* p, int32_t* out, int32_t n) {
  if (p == nullptr || (out == nullptr && n > 0)) return RKV_ERR_NULL;
  if (n < 0 || n > (int32_t)p->table.size()) return RKV_ERR_ARG;
  for (int32_t i = 0; i < n; ++i) out[i] = p->table[(size_t)i];
  return RKV_OK;
}

int32_t rkv_pager_reserve(rkv_pager* p, int32_t n, int32_t* first_chunk, int32_t* n_new,
                          int32_t* slots) {
  if (p == nullptr || first_chunk == nullptr || n_new == nullptr || slots == nullptr)
    return RKV_ERR_NULL;
  if (p->pending || n < 1 || n > RKV_MAX_APPEND) return RKV_ERR_ARG;
  const int64_t c0 = ceil_chunks(p->ctx);              // first chunk holding no position yet
  const int64_t c1 = ceil_chunks(p->ctx + n);          // chunks needed after the block
  if (c1 > (int64_t)p->table.size()) return RKV_ERR_TABLE;
  const int32_t k = (int32_t)(c1 - c0);
  if (k > (int32_t)p->free.size()) return RKV_ERR_TABLE;
  for (int32_t i = 0; i < k; ++i) {
    const int32_t s = p->free.back();
    p->free.pop_back();
    p->table[(size_t)(c0 + i)] = s;
    slots[i] = s;
  }
  p->pending = true;
  p->pend_n = n;
  p->pend_first = (int32_t)c0;
  p->pend_new = k;
  *first_chunk = (int32_t)c0;
  *n_new = k;
  return RKV_OK;
}

int32_t rkv_pager_commit(rkv_pager* p, int32_t n_keep) {
  if (p == nullptr) return RKV_ERR_NULL;
  if (!p->pending || n_keep < 0 || n_keep > p->pend_n) return RKV_ERR_ARG;
  p->ctx += n_keep;
  const int64_t keep_chunks = ceil_chunks(p->ctx);
  // the block's chunks past the committed length, last first, so that the earliest of them
  // is the next one handed out again
  for (int32_t i = p->pend_new - 1; i >= 0; --i) {
    const int64_t c = (int64_t)p->pend_first + i;
    if (c < keep_chunks) break;
    p->free.push_back(p->table[(size_t)c]);
    p->table[(size_t)c] = -1;
  }
  p->pending = false;
  p->pend_n = p->pend_first = p->pend_new = 0;
  return RKV_OK;
}

int32_t rkv_pager_evict(rkv_pager* p, const int32_t* chunk_ids, int32_t n, int32_t* slots) {
  if (p == nullptr || ((chunk_ids == nullptr || slots == nullptr) && n > 0)) return RKV_ERR_NULL;
  if (n < 0) return RKV_ERR_ARG;
  const int64_t full = p->ctx / kChunk;             // chunks whose 64 positions are committed
  std::vector<int32_t> seen(chunk_ids, chunk_ids + n);
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) return RKV_ERR_ARG;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t c = chunk_ids[i];
    if (c < 0 || c >= full || p->table[(size_t)c] < 0) return RKV_ERR_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {
    const size_t c = (size_t)chunk_ids[i];
    slots[i] = p->table[c];
    p->free.push_back(p->table[c]);
    p->table[c] = RKV_PAGED_OUT;
  }
  return RKV_OK;
}

int32_t rkv_pager_restore(rkv_pager* p, const int32_t* chunk_ids, int32_t n, int32_t* slots) {
  if (p == nullptr || ((chunk_ids == nullptr || slots == nullptr) && n > 0)) return RKV_ERR_NULL;
  if (n < 0) return RKV_ERR_ARG;
  std::vector<int32_t> seen(chunk_ids, chunk_ids + n);
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) return RKV_ERR_ARG;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t c = chunk_ids[i];
    if (c < 0 || c >= (int32_t)p->table.size() || p->table[(size_t)c] != RKV_PAGED_OUT)
      return RKV_ERR_ARG;
  }
  if (n > (int32_t)p->free.size()) return RKV_ERR_TABLE;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = p->free.back();
    p->free.pop_back();
    p->table[(size_t)chunk_ids[i]] = s;
    slots[i] = s;
  }
  return RKV_OK;
}

int32_t rkv_pager_resident(const rkv_pager* p, int32_t* chunk_ids, int32_t* slots, int32_t cap) {
  if (p == nullptr) return RKV_ERR_NULL;
  if (cap < 0) return RKV_ERR_ARG;
  if (cap > 0 && (chunk_ids == nullptr || slots == nullptr)) return RKV_ERR_NULL;
  int32_t k = 0;
  for (size_t c = 0; c < p->table.size(); ++c) {
    if (p->table[c] < 0) continue;
    if (k < cap) {
      chunk_ids[k] = (int32_t)c;
      slots[k] = p->table[c];
    }
    ++k;
  }
  return k;
}

}  // extern "C"
