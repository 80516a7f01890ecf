// The C entry points of libring_kv: argument checks (host only, before any HIP call), the
// split of the key range, workspace carving, and kernel launches on the caller's stream.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/ring_kv.h"
#include "rkv_launch.hpp"

namespace rkv {

// The verify kernels run one workgroup per compute unit (each takes a unit's LDS or registers),
// so split counts and row tiles are chosen from the device's unit count: 256 on a whole MI355X,
// fewer on a partitioned one.  Cached per device; the fallback is a whole MI355X.
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  constexpr int kDefault = 256;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kDefault;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = kDefault;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace rkv

namespace {

using rkv::ChunkAttnArgs;

constexpr int kChunk = RKV_CHUNK;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int32_t check_dims(const rkv_attn_dims* d) {
  if (d == nullptr) return RKV_ERR_NULL;
  if (d->q_len < 1 || d->n_kv_heads < 1 || d->n_q_heads < 1) return RKV_ERR_SHAPE;
  if (d->n_q_heads % d->n_kv_heads != 0) return RKV_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return RKV_ERR_SHAPE;
  if ((int64_t)d->q_len * (d->n_q_heads / d->n_kv_heads) > RKV_MAX_ROWS) return RKV_ERR_SHAPE;
  if (!(d->scale >= 0.f) || isinf(d->scale)) return RKV_ERR_ARG;
  if (d->dtype != RKV_F32 && d->dtype != RKV_BF16) return RKV_ERR_DTYPE;
  return RKV_OK;
}

float scale_log2(const rkv_attn_dims* d) {
  const float sc = d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->head_dim);
  return sc * 1.4426950408889634f;
}

int rows_of(const rkv_attn_dims* d) { return d->q_len * (d->n_q_heads / d->n_kv_heads); }

enum Store { kContig, kRing, kPaged };

// Split count the automatic choice aims at: about one workgroup per compute unit over all
// (KV head, row tile) pairs.  A prefill block over the ring is the exception: its row tiles
// fill the chip by themselves and each sees only a window of keys, so it is not split.
int64_t auto_split_target(const rkv_attn_dims* d, Store store) {
  const int rows = rows_of(d);
  const bool prefill = store != kContig && rows > rkv::kVerifyMaxRows;
  if (prefill && store == kRing) return 1;
  const int tile = prefill ? rkv::kPrefillTileRows : 64;
  const int64_t units = (int64_t)d->n_kv_heads * ((rows + tile - 1) / tile);
  return (rkv::device_cu_count() + units - 1) / units;
}

// The paged store's automatic split target for a context of n_chunks chunks.  A verify block's
// merge reads one partial per split and row, so below about 256 chunks fewer, longer splits win:
// at least n_chunks / 4 and half the fill target, never more than the chunks (one chunk per split
// keeps its single-round-trip path) nor the fill target.  Measured in graph replay (16 query / 4
// KV heads): 4,096 positions 13.2 -> 12.4 us, 8,192: 15.5 -> 14.3 us, 12,288: 17.0 -> 15.7 us;
// from 16,384 positions on the fill target stays best.  Monotone in n_chunks.  Prefill blocks keep
// the fill target.
int64_t paged_split_target(const rkv_attn_dims* d, int64_t n_chunks) {
  const int64_t t = auto_split_target(d, kPaged);
  if (rows_of(d) > rkv::kVerifyMaxRows) return t;
  const int64_t half = t / 2 > 1 ? t / 2 : 1;
  const int64_t lo = n_chunks < half ? n_chunks : half;
  const int64_t quarter = (n_chunks + 3) / 4;
  const int64_t want = lo > quarter ? lo : quarter;
  return want < t ? want : t;
}

// Split n_chunks whole chunks into ranges: num_splits <= 0 asks for `target` splits.  Returns
// the split count actually used (no empty split unless the caller asked for more splits than
// chunks) and the chunks per split.
void choose_splits(int64_t n_chunks, int64_t target, int32_t requested, int32_t* splits,
                   int32_t* cps) {
  if (n_chunks <= 0) { *splits = 1; *cps = 1; return; }
  if (requested > 0) {
    *splits = requested;
    *cps = (int32_t)((n_chunks + requested - 1) / requested);
    return;
  }
  int64_t s = target;
  if (s > n_chunks) s = n_chunks;
  if (s < 1) s = 1;
  const int64_t c = (n_chunks + s - 1) / s;
  *cps = (int32_t)c;
  *splits = (int32_t)((n_chunks + c - 1) / c);
}

// Splits for n_chunks when the workspace was sized for n_max >= n_chunks chunks: never more
// splits than that workspace holds.
void split_within(int64_t n_chunks, int64_t n_max, int64_t target, int32_t requested,
                  int32_t* splits, int32_t* cps) {
  int32_t s_max, c_max;
  choose_splits(n_max, target, requested, &s_max, &c_max);
  choose_splits(n_chunks, target, requested, splits, cps);
  if (*splits > s_max) {
    *splits = s_max;
    *cps = (int32_t)((n_chunks + s_max - 1) / s_max);
  }
}

size_t partial_bytes(const rkv_attn_dims* d, int32_t splits) {
  if (splits <= 1) return 0;
  const size_t prow = (size_t)d->n_kv_heads * splits * rows_of(d);
  return align_up(prow * d->head_dim * sizeof(float)) + align_up(prow * sizeof(float));
}

void carve(void* ws, const rkv_attn_dims* d, int32_t splits, float** po, float** pl) {
  const size_t prow = (size_t)d->n_kv_heads * splits * rows_of(d);
  *po = static_cast<float*>(ws);
  *pl = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(prow * d->head_dim * sizeof(float)));
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? RKV_OK : RKV_ERR_HIP; }

// The row copies into the chunked stores move 16-byte pieces.
bool aligned16(const void* a, const void* b, const void* c, const void* d) {
  return (((uintptr_t)a | (uintptr_t)b | (uintptr_t)c | (uintptr_t)d) & 15) == 0;
}

// ws: where the partials go; tickets: the counters of the one-launch ring layer (nullptr: the
// partials are merged by a second launch)
int32_t run_chunk_attn(ChunkAttnArgs& a, const rkv_attn_dims* d, void* ws, int32_t* tickets,
                       float* out, float* lse, hipStream_t st) {
  if (a.cps > rkv::kMaxSplitChunks) return RKV_ERR_SHAPE;
  a.out = out;
  a.lse = lse;
  a.part_o = a.part_lse = nullptr;
  a.tickets = tickets;
  a.fill_wgs = rkv::device_cu_count();
  if (a.num_splits > 1) carve(ws, d, a.num_splits, &a.part_o, &a.part_lse);
  bool merged = false;
  hipError_t e = rkv::launch_chunk_attn(a, st, &merged);
  if (e != hipSuccess || a.num_splits == 1 || merged) return hip_status(e);
  rkv::MergeArgs m{a.part_o, a.part_lse, out, lse, a.q_len, a.G, a.n_q_heads, a.n_kv_heads,
                   a.head_dim, a.num_splits};
  return hip_status(rkv::launch_merge(m, st));
}

ChunkAttnArgs paged_args(const rkv_attn_dims* d, const void* q, const void* k, const void* v,
                         const int32_t* pt, int32_t n_slots, int64_t ctx_len) {
  ChunkAttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.pt = pt;
  a.n_slots = n_slots;
  a.q_len = d->q_len;
  a.G = d->n_q_heads / d->n_kv_heads;
  a.n_q_heads = d->n_q_heads;
  a.n_kv_heads = d->n_kv_heads;
  a.head_dim = d->head_dim;
  a.p0 = ctx_len - d->q_len;
  a.window = 0;
  a.valid_lo = 0;
  a.valid_hi = ctx_len;
  a.c_first = 0;
  a.n_chunks = (ctx_len + kChunk - 1) / kChunk;
  a.scale_log2 = scale_log2(d);
  return a;
}

int32_t check_paged(const rkv_attn_dims* d, const void* q, const void* k, const void* v,
                    const int32_t* pt, int32_t n_table, int32_t n_slots, int32_t chunk_size,
                    int64_t ctx_len) {
  int32_t st = check_dims(d);
  if (st != RKV_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || pt == nullptr) return RKV_ERR_NULL;
  if (d->dtype != RKV_BF16) return RKV_ERR_DTYPE;
  if (ctx_len < d->q_len) return RKV_ERR_SHAPE;
  if (chunk_size != kChunk || n_slots < 1) return RKV_ERR_TABLE;
  if ((int64_t)n_table * kChunk < ctx_len) return RKV_ERR_TABLE;
  if ((ctx_len + kChunk - 1) / kChunk > INT32_MAX) return RKV_ERR_TABLE;
  return RKV_OK;
}

int32_t check_ring(const rkv_attn_dims* d, const void* q, const void* k, const void* v,
                   int64_t pos0, int32_t ring_head, int32_t ring_size, int32_t window) {
  int32_t st = check_dims(d);
  if (st != RKV_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr) return RKV_ERR_NULL;
  if (d->dtype != RKV_BF16) return RKV_ERR_DTYPE;
  if (pos0 < 0 || window < 1) return RKV_ERR_ARG;
  if (ring_size < kChunk || ring_size % kChunk != 0) return RKV_ERR_RING;
  if ((int64_t)ring_size < (int64_t)window + d->q_len - 1) return RKV_ERR_RING;
  if (ring_head < 0 || ring_head != (int32_t)(pos0 % ring_size)) return RKV_ERR_RING;
  return RKV_OK;
}

}  // namespace

extern "C" {

int32_t rkv_abi_version(void) { return RKV_ABI_VERSION; }

const char* rkv_status_str(int32_t status) {
  switch (status) {
    case RKV_OK: return "ok";
    case RKV_ERR_NULL: return "a required pointer is NULL";
    case RKV_ERR_SHAPE: return "head counts, head_dim, q_len or ctx_len out of range";
    case RKV_ERR_DTYPE: return "dtype not supported by this call";
    case RKV_ERR_RING: return "ring size, window or head pointer inconsistent";
    case RKV_ERR_TABLE: return "chunk size unsupported or page table / pool too small";
    case RKV_ERR_WORKSPACE: return "workspace missing or too small";
    case RKV_ERR_HIP: return "HIP launch failed";
    case RKV_ERR_ARG: return "argument out of range";
    default: return "unknown status";
  }
}

// ---- contiguous reference layout ---------------------------------------------------------

static void contig_range(const rkv_attn_dims* d, int64_t ctx_len, int32_t window,
                         int64_t* c_first, int64_t* n_chunks) {
  const int64_t p0 = ctx_len - d->q_len;
  const int64_t lo = window > 0 ? (p0 - window + 1 > 0 ? p0 - window + 1 : 0) : 0;
  *c_first = lo / kChunk;
  *n_chunks = (ctx_len + kChunk - 1) / kChunk - *c_first;
}

size_t decode_attn_ref_layout_workspace_bytes(const rkv_attn_dims* dims, int64_t ctx_len,
                                              int32_t num_splits) {
  if (check_dims(dims) != RKV_OK || ctx_len < dims->q_len || num_splits < 0) return 0;
  int64_t c_first, n_chunks;
  contig_range(dims, ctx_len, 0, &c_first, &n_chunks);
  int32_t s, cps;
  choose_splits(n_chunks, auto_split_target(dims, kContig), num_splits, &s, &cps);
  return partial_bytes(dims, s);
}

int32_t decode_attn_ref_layout(const rkv_attn_dims* dims, const void* q, const void* k,
                               const void* v, int64_t ctx_len, int32_t window,
                               int32_t num_splits, void* workspace, size_t workspace_bytes,
                               float* out, float* lse, void* stream) {
  int32_t st = check_dims(dims);
  if (st != RKV_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return RKV_ERR_NULL;
  if (ctx_len < dims->q_len) return RKV_ERR_SHAPE;
  if (window < 0 || num_splits < 0) return RKV_ERR_ARG;
  int64_t c_first, n_chunks, c0, nfull;
  contig_range(dims, ctx_len, window, &c_first, &n_chunks);
  contig_range(dims, ctx_len, 0, &c0, &nfull);
  int32_t s, cps;
  split_within(n_chunks, nfull, auto_split_target(dims, kContig), num_splits, &s, &cps);
  if (s > 1 && (workspace == nullptr || workspace_bytes < partial_bytes(dims, s)))
    return RKV_ERR_WORKSPACE;
  rkv::ContigArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.dtype = dims->dtype;
  a.q_len = dims->q_len;
  a.G = dims->n_q_heads / dims->n_kv_heads;
  a.n_q_heads = dims->n_q_heads;
  a.n_kv_heads = dims->n_kv_heads;
  a.head_dim = dims->head_dim;
  a.ctx_len = ctx_len;
  a.window = window;
  a.c_first = c_first;
  a.n_chunks = n_chunks;
  a.cps = cps;
  a.num_splits = s;
  a.scale_log2 = scale_log2(dims);
  a.out = out;
  a.lse = lse;
  if (s > 1) carve(workspace, dims, s, &a.part_o, &a.part_lse);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = rkv::launch_contig_attn(a, hs);
  if (e != hipSuccess || s == 1) return hip_status(e);
  rkv::MergeArgs m{a.part_o, a.part_lse, out, lse, a.q_len, a.G, a.n_q_heads, a.n_kv_heads,
                   a.head_dim, s};
  return hip_status(rkv::launch_merge(m, hs));
}

// ---- sliding-window ring -----------------------------------------------------------------

static void ring_range(const rkv_attn_dims* d, int64_t pos0, int32_t window, int64_t* c_first,
                       int64_t* n_chunks) {
  const int64_t lo = pos0 - window + 1 > 0 ? pos0 - window + 1 : 0;
  const int64_t hi = pos0 + d->q_len - 1;
  *c_first = lo / kChunk;
  *n_chunks = hi / kChunk - lo / kChunk + 1;
}

// chunks the widest window span can touch, whatever pos0 is
static int64_t ring_max_chunks(const rkv_attn_dims* d, int32_t window) {
  const int64_t span = (int64_t)window + d->q_len - 1;
  return (span + kChunk - 2) / kChunk + 1;
}

// A ring call's workspace: kTicketBytes of counters (zero before the workspace's first use; every
// call leaves its arrival counters zero), then the partials of the widest span's split layout.
static size_t ring_workspace_full(const rkv_attn_dims* dims, int32_t window, int32_t num_splits) {
  int32_t s, cps;
  choose_splits(ring_max_chunks(dims, window), auto_split_target(dims, kRing), num_splits, &s,
                &cps);
  return s > 1 ? rkv::kTicketBytes + partial_bytes(dims, s) : 0;
}

// Where a ring call's partials and counters go.  A workspace of the full size holds the counters
// first and the partials after them (one launch where the kernel supports it); a smaller one
// that still holds this call's partials gets them at its start and no counters (the partials
// are merged by a second launch).
static int32_t ring_workspace(const rkv_attn_dims* dims, int32_t window, int32_t num_splits,
                              int32_t s, void* ws, size_t bytes, void** part_ws,
                              int32_t** tickets) {
  *part_ws = ws;
  *tickets = nullptr;
  if (s <= 1) return RKV_OK;
  if (ws == nullptr || bytes < partial_bytes(dims, s)) return RKV_ERR_WORKSPACE;
  const size_t full = ring_workspace_full(dims, window, num_splits);
  if (full > 0 && bytes >= full) {
    *tickets = static_cast<int32_t*>(ws);
    *part_ws = static_cast<char*>(ws) + rkv::kTicketBytes;
  }
  return RKV_OK;
}

size_t verify_attn_ring_workspace_bytes(const rkv_attn_dims* dims, int32_t ring_size,
                                        int32_t window, int32_t num_splits) {
  if (check_dims(dims) != RKV_OK || window < 1 || num_splits < 0 || ring_size < kChunk) return 0;
  return ring_workspace_full(dims, window, num_splits);
}

int32_t verify_attn_ring(const rkv_attn_dims* dims, const void* q, const void* k_ring,
                         const void* v_ring, int64_t pos0, int32_t ring_head,
                         int32_t ring_size, int32_t window, int32_t num_splits,
                         void* workspace, size_t workspace_bytes, float* out, float* lse,
                         void* stream) {
  int32_t st = check_ring(dims, q, k_ring, v_ring, pos0, ring_head, ring_size, window);
  if (st != RKV_OK) return st;
  if (out == nullptr) return RKV_ERR_NULL;
  if (num_splits < 0) return RKV_ERR_ARG;
  int64_t c_first, n_chunks;
  ring_range(dims, pos0, window, &c_first, &n_chunks);
  int32_t s, cps;
  split_within(n_chunks, ring_max_chunks(dims, window), auto_split_target(dims, kRing),
               num_splits, &s, &cps);
  void* part_ws;
  int32_t* tickets;
  st = ring_workspace(dims, window, num_splits, s, workspace, workspace_bytes, &part_ws, &tickets);
  if (st != RKV_OK) return st;
  ChunkAttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_ring);
  a.v = static_cast<const uint16_t*>(v_ring);
  a.pt = nullptr;
  a.n_slots = ring_size / kChunk;
  a.q_len = dims->q_len;
  a.G = dims->n_q_heads / dims->n_kv_heads;
  a.n_q_heads = dims->n_q_heads;
  a.n_kv_heads = dims->n_kv_heads;
  a.head_dim = dims->head_dim;
  a.p0 = pos0;
  a.window = window;
  const int64_t end = pos0 + dims->q_len;
  a.valid_lo = end - ring_size > 0 ? end - ring_size : 0;
  a.valid_hi = end;
  a.c_first = c_first;
  a.n_chunks = n_chunks;
  a.cps = cps;
  a.num_splits = s;
  a.scale_log2 = scale_log2(dims);
  return run_chunk_attn(a, dims, part_ws, tickets, out, lse, static_cast<hipStream_t>(stream));
}

// ---- paged pool --------------------------------------------------------------------------

int32_t verify_attn_paged_auto_splits(const rkv_attn_dims* dims, int64_t ctx_len,
                                      int32_t chunk_size) {
  if (check_dims(dims) != RKV_OK || chunk_size != kChunk || ctx_len < 1) return 0;
  int32_t s, cps;
  const int64_t n = (ctx_len + kChunk - 1) / kChunk;
  choose_splits(n, paged_split_target(dims, n), 0, &s, &cps);
  return s;
}

size_t verify_attn_paged_workspace_bytes(const rkv_attn_dims* dims, int64_t ctx_len,
                                         int32_t chunk_size, int32_t num_splits) {
  if (check_dims(dims) != RKV_OK || chunk_size != kChunk || ctx_len < dims->q_len ||
      num_splits < 0)
    return 0;
  int32_t s, cps;
  const int64_t n = (ctx_len + kChunk - 1) / kChunk;
  choose_splits(n, paged_split_target(dims, n), num_splits, &s, &cps);
  return partial_bytes(dims, s);
}

int32_t verify_attn_paged(const rkv_attn_dims* dims, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* page_table, int32_t n_table,
                          int32_t n_slots, int32_t chunk_size, int64_t ctx_len,
                          int32_t num_splits, void* workspace, size_t workspace_bytes,
                          float* out, float* lse, void* stream) {
  int32_t st = check_paged(dims, q, k_pool, v_pool, page_table, n_table, n_slots, chunk_size,
                           ctx_len);
  if (st != RKV_OK) return st;
  if (out == nullptr) return RKV_ERR_NULL;
  if (num_splits < 0) return RKV_ERR_ARG;
  ChunkAttnArgs a = paged_args(dims, q, k_pool, v_pool, page_table, n_slots, ctx_len);
  choose_splits(a.n_chunks, paged_split_target(dims, a.n_chunks), num_splits, &a.num_splits,
                &a.cps);
  if (a.num_splits > 1 &&
      (workspace == nullptr || workspace_bytes < partial_bytes(dims, a.num_splits)))
    return RKV_ERR_WORKSPACE;
  return run_chunk_attn(a, dims, workspace, nullptr, out, lse, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Split partials of verify_attn_paged_noalloc: a file-scope device array, one copy per device the
// library runs on, held until the process ends.  Its name is a host-side stand-in in host code;
// kernels get the device address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = RKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on the current device, looked up once per device (with that
// device current); nullptr if the lookup fails.
void* scratch_address() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

int32_t verify_attn_paged_noalloc(const rkv_attn_dims* dims, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* page_table, int32_t n_table,
                                  int32_t n_slots, int32_t chunk_size, int64_t ctx_len,
                                  int32_t num_splits, float* out, float* lse, void* stream) {
  int32_t st = check_paged(dims, q, k_pool, v_pool, page_table, n_table, n_slots, chunk_size,
                           ctx_len);
  if (st != RKV_OK) return st;
  if (out == nullptr) return RKV_ERR_NULL;
  if (num_splits < 0) return RKV_ERR_ARG;
  ChunkAttnArgs a = paged_args(dims, q, k_pool, v_pool, page_table, n_slots, ctx_len);
  choose_splits(a.n_chunks, paged_split_target(dims, a.n_chunks), num_splits, &a.num_splits,
                &a.cps);
  if (a.num_splits > 1 && partial_bytes(dims, a.num_splits) > kScratchBytes)
    return RKV_ERR_WORKSPACE;
  void* ws = nullptr;
  if (a.num_splits > 1 && (ws = scratch_address()) == nullptr) return RKV_ERR_HIP;
  return run_chunk_attn(a, dims, ws, nullptr, out, lse, static_cast<hipStream_t>(stream));
}

int32_t verify_attn_paged_resident(const rkv_attn_dims* dims, const void* q,
                                   const void* k_pool, const void* v_pool,
                                   const int32_t* d_slots, const int32_t* chunk_ids,
                                   int32_t n_res, int32_t n_slots, int64_t ctx_len,
                                   int32_t num_splits, void* workspace, size_t workspace_bytes,
                                   float* out, float* lse, void* stream) {
  int32_t st = check_dims(dims);
  if (st != RKV_OK) return st;
  if (chunk_ids == nullptr) return RKV_ERR_NULL;
  if (ctx_len < dims->q_len) return RKV_ERR_SHAPE;
  if (n_res < 1) return RKV_ERR_TABLE;
  for (int32_t i = 0; i < n_res; ++i)
    if (chunk_ids[i] < 0 || (i > 0 && chunk_ids[i] <= chunk_ids[i - 1])) return RKV_ERR_TABLE;
  // the block's chunks must close the list, in order
  const int64_t first = (ctx_len - dims->q_len) / kChunk;
  const int64_t last = (ctx_len - 1) / kChunk;
  const int64_t nb = last - first + 1;
  if (nb > n_res) return RKV_ERR_TABLE;
  for (int64_t j = 0; j < nb; ++j)
    if (chunk_ids[n_res - nb + j] != first + j) return RKV_ERR_TABLE;
  // every listed chunk before the block's first is wholly visible: the packed list is a page
  // table at a context shorter by the chunks that are not listed
  const int64_t missing = first - (n_res - nb);
  return verify_attn_paged(dims, q, k_pool, v_pool, d_slots, n_res, n_slots, kChunk,
                           ctx_len - kChunk * missing, num_splits, workspace, workspace_bytes,
                           out, lse, stream);
}

int32_t verify_attn_paged_partial(const rkv_attn_dims* dims, const void* q,
                                  const void* k_pool, const void* v_pool,
                                  const int32_t* page_table, int32_t n_table, int32_t n_slots,
                                  int32_t chunk_size, int64_t ctx_len, int32_t num_splits,
                                  float* part_out, float* part_lse, void* stream) {
  int32_t st = check_paged(dims, q, k_pool, v_pool, page_table, n_table, n_slots, chunk_size,
                           ctx_len);
  if (st != RKV_OK) return st;
  if (part_out == nullptr || part_lse == nullptr) return RKV_ERR_NULL;
  if (num_splits < 1) return RKV_ERR_ARG;
  ChunkAttnArgs a = paged_args(dims, q, k_pool, v_pool, page_table, n_slots, ctx_len);
  a.num_splits = num_splits;
  a.cps = (int32_t)((a.n_chunks + num_splits - 1) / num_splits);
  if (a.cps < 1) a.cps = 1;
  if (a.cps > rkv::kMaxSplitChunks) return RKV_ERR_SHAPE;
  a.part_o = part_out;     // partial layout even for one split
  a.part_lse = part_lse;
  a.fill_wgs = rkv::device_cu_count();
  bool merged = false;
  return hip_status(rkv::launch_chunk_attn(a, static_cast<hipStream_t>(stream), &merged));
}

// ---- one captured step replayed across decode steps: the block position on the device ----

// The block's own rows for the calls that append them in the attention launch: both given, and
// every pointer 16-byte aligned (the rows move as 16-byte pieces).
static int32_t new_rows_check(const void* k_new, const void* v_new, const void* k, const void* v) {
  if (k_new == nullptr || v_new == nullptr || k == nullptr || v == nullptr) return RKV_ERR_NULL;
  if (!aligned16(k_new, v_new, k, v)) return RKV_ERR_ARG;
  return RKV_OK;
}

static void set_new_rows(ChunkAttnArgs& a, const void* k_new, const void* v_new, const void* k,
                         const void* v) {
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.k_w = k_new != nullptr ? static_cast<uint16_t*>(const_cast<void*>(k)) : nullptr;
  a.v_w = k_new != nullptr ? static_cast<uint16_t*>(const_cast<void*>(v)) : nullptr;
}

// The ring and pool calls at a device-resident position; k_new, v_new (both or neither): the
// block's own rows, appended by the same launch.
static int32_t ring_dev(const rkv_attn_dims* dims, const void* q, const void* k_new,
                        const void* v_new, const void* k_ring, const void* v_ring,
                        const int64_t* d_pos, int64_t pos_cap, int32_t ring_size, int32_t window,
                        int32_t num_splits, void* workspace, size_t workspace_bytes, float* out,
                        float* lse, void* stream) {
  int32_t st = check_ring(dims, q, k_ring, v_ring, 0, 0, ring_size, window);
  if (st != RKV_OK) return st;
  if (d_pos == nullptr || out == nullptr) return RKV_ERR_NULL;
  if (rows_of(dims) > rkv::kVerifyMaxRows) return RKV_ERR_SHAPE;
  if (pos_cap < 0 || num_splits < 0) return RKV_ERR_ARG;
  // the split layout covers the widest span any position can have
  const int64_t n_max = ring_max_chunks(dims, window);
  int32_t s, cps;
  choose_splits(n_max, auto_split_target(dims, kRing), num_splits, &s, &cps);
  void* part_ws;
  int32_t* tickets;
  st = ring_workspace(dims, window, num_splits, s, workspace, workspace_bytes, &part_ws, &tickets);
  if (st != RKV_OK) return st;
  ChunkAttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_ring);
  a.v = static_cast<const uint16_t*>(v_ring);
  a.pt = nullptr;
  a.n_slots = ring_size / kChunk;
  a.q_len = dims->q_len;
  a.G = dims->n_q_heads / dims->n_kv_heads;
  a.n_q_heads = dims->n_q_heads;
  a.n_kv_heads = dims->n_kv_heads;
  a.head_dim = dims->head_dim;
  a.window = window;
  a.n_chunks = n_max;
  a.cps = cps;
  a.num_splits = s;
  a.scale_log2 = scale_log2(dims);
  a.d_pos = d_pos;
  a.pos_cap = pos_cap;
  a.ring_size = ring_size;
  set_new_rows(a, k_new, v_new, k_ring, v_ring);
  return run_chunk_attn(a, dims, part_ws, tickets, out, lse, static_cast<hipStream_t>(stream));
}

static int32_t paged_dev(const rkv_attn_dims* dims, const void* q, const void* k_new,
                         const void* v_new, const void* k_pool, const void* v_pool,
                         const int32_t* page_table, int32_t n_table, int32_t n_slots,
                         int32_t chunk_size, const int64_t* d_pos, int64_t pos_cap,
                         int32_t num_splits, void* workspace, size_t workspace_bytes, float* out,
                         float* lse, void* stream) {
  if (dims == nullptr) return RKV_ERR_NULL;
  if (pos_cap < 0 || pos_cap > INT64_MAX / 2) return RKV_ERR_ARG;
  const int64_t ctx_max = pos_cap + dims->q_len;
  int32_t st = check_paged(dims, q, k_pool, v_pool, page_table, n_table, n_slots, chunk_size,
                           ctx_max);
  if (st != RKV_OK) return st;
  if (d_pos == nullptr || out == nullptr) return RKV_ERR_NULL;
  if (rows_of(dims) > rkv::kVerifyMaxRows) return RKV_ERR_SHAPE;
  if (num_splits < 0) return RKV_ERR_ARG;
  // the split layout is that of the largest context the position can reach
  ChunkAttnArgs a = paged_args(dims, q, k_pool, v_pool, page_table, n_slots, ctx_max);
  choose_splits(a.n_chunks, paged_split_target(dims, a.n_chunks), num_splits, &a.num_splits,
                &a.cps);
  if (a.num_splits > 1 &&
      (workspace == nullptr || workspace_bytes < partial_bytes(dims, a.num_splits)))
    return RKV_ERR_WORKSPACE;
  a.d_pos = d_pos;
  a.pos_cap = pos_cap;
  set_new_rows(a, k_new, v_new, k_pool, v_pool);
  return run_chunk_attn(a, dims, workspace, nullptr, out, lse, static_cast<hipStream_t>(stream));
}

int32_t verify_attn_ring_dev(const rkv_attn_dims* dims, const void* q, const void* k_ring,
                             const void* v_ring, const int64_t* d_pos, int64_t pos_cap,
                             int32_t ring_size, int32_t window, int32_t num_splits,
                             void* workspace, size_t workspace_bytes, float* out, float* lse,
                             void* stream) {
  return ring_dev(dims, q, nullptr, nullptr, k_ring, v_ring, d_pos, pos_cap, ring_size, window,
                  num_splits, workspace, workspace_bytes, out, lse, stream);
}

int32_t verify_attn_paged_dev(const rkv_attn_dims* dims, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* page_table, int32_t n_table,
                              int32_t n_slots, int32_t chunk_size, const int64_t* d_pos,
                              int64_t pos_cap, int32_t num_splits, void* workspace,
                              size_t workspace_bytes, float* out, float* lse, void* stream) {
  return paged_dev(dims, q, nullptr, nullptr, k_pool, v_pool, page_table, n_table, n_slots,
                   chunk_size, d_pos, pos_cap, num_splits, workspace, workspace_bytes, out, lse,
                   stream);
}

int32_t verify_attn_ring_append_dev(const rkv_attn_dims* dims, const void* q, const void* k_new,
                                    const void* v_new, void* k_ring, void* v_ring,
                                    const int64_t* d_pos, int64_t pos_cap, int32_t ring_size,
                                    int32_t window, int32_t num_splits, void* workspace,
                                    size_t workspace_bytes, float* out, float* lse, void* stream) {
  int32_t st = new_rows_check(k_new, v_new, k_ring, v_ring);
  if (st != RKV_OK) return st;
  return ring_dev(dims, q, k_new, v_new, k_ring, v_ring, d_pos, pos_cap, ring_size, window,
                  num_splits, workspace, workspace_bytes, out, lse, stream);
}

int32_t verify_attn_paged_append_dev(const rkv_attn_dims* dims, const void* q, const void* k_new,
                                     const void* v_new, void* k_pool, void* v_pool,
                                     const int32_t* page_table, int32_t n_table, int32_t n_slots,
                                     int32_t chunk_size, const int64_t* d_pos, int64_t pos_cap,
                                     int32_t num_splits, void* workspace, size_t workspace_bytes,
                                     float* out, float* lse, void* stream) {
  int32_t st = new_rows_check(k_new, v_new, k_pool, v_pool);
  if (st != RKV_OK) return st;
  return paged_dev(dims, q, k_new, v_new, k_pool, v_pool, page_table, n_table, n_slots,
                   chunk_size, d_pos, pos_cap, num_splits, workspace, workspace_bytes, out, lse,
                   stream);
}

int32_t attn_merge_partials(const rkv_attn_dims* dims, int32_t num_splits,
                            const float* part_out, const float* part_lse, float* out,
                            float* lse, void* stream) {
  if (dims == nullptr) return RKV_ERR_NULL;
  rkv_attn_dims d = *dims;
  d.dtype = RKV_BF16;
  int32_t st = check_dims(&d);
  if (st != RKV_OK) return st;
  if (part_out == nullptr || part_lse == nullptr || out == nullptr) return RKV_ERR_NULL;
  if (num_splits < 1) return RKV_ERR_ARG;
  rkv::MergeArgs m{part_out, part_lse, out, lse, d.q_len, d.n_q_heads / d.n_kv_heads,
                   d.n_q_heads, d.n_kv_heads, d.head_dim, num_splits};
  return hip_status(rkv::launch_merge(m, static_cast<hipStream_t>(stream)));
}

// ---- greedy accept -----------------------------------------------------------------------

static void accept_parts(int32_t vocab, int32_t* parts, int32_t* part_len) {
  // about 4096 logits (16 KiB) per workgroup
  int32_t pl = 4096;
  if (vocab < pl) pl = (vocab + 3) / 4 * 4;
  if (pl < 4) pl = 4;
  *part_len = pl;
  *parts = (vocab + pl - 1) / pl;
}

size_t verify_accept_workspace_bytes(int32_t n_draft, int32_t vocab) {
  if (n_draft < 0 || n_draft > 255 || vocab < 1) return 0;
  int32_t parts, pl;
  accept_parts(vocab, &parts, &pl);
  const size_t n = (size_t)(n_draft + 1) * parts;
  return align_up(n * sizeof(float)) + align_up(n * sizeof(int32_t));
}

int32_t verify_accept(const float* logits, int32_t n_draft, int32_t vocab,
                      const int32_t* proposals, int32_t* accept_len, int32_t* committed,
                      int32_t* row_argmax, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (logits == nullptr || accept_len == nullptr || committed == nullptr) return RKV_ERR_NULL;
  if (n_draft > 0 && proposals == nullptr) return RKV_ERR_NULL;
  if (n_draft < 0 || n_draft > 255 || vocab < 1) return RKV_ERR_SHAPE;
  const size_t need = verify_accept_workspace_bytes(n_draft, vocab);
  if (workspace == nullptr || workspace_bytes < need) return RKV_ERR_WORKSPACE;
  rkv::AcceptArgs a{};
  a.logits = logits;
  a.n_rows = n_draft + 1;
  a.vocab = vocab;
  a.proposals = proposals;
  a.accept_len = accept_len;
  a.committed = committed;
  a.row_argmax = row_argmax;
  accept_parts(vocab, &a.parts, &a.part_len);
  const size_t n = (size_t)a.n_rows * a.parts;
  a.part_val = static_cast<float*>(workspace);
  a.part_idx = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align_up(n * sizeof(float)));
  return hip_status(rkv::launch_accept(a, static_cast<hipStream_t>(stream)));
}

// ---- layout helpers ----------------------------------------------------------------------

int32_t ref_layout_to_ring(const void* k_src, const void* v_src, int64_t pos_first, int64_t n,
                           int32_t n_kv_heads, int32_t head_dim, int32_t dtype, void* k_ring,
                           void* v_ring, int32_t ring_size, void* stream) {
  if (k_src == nullptr || v_src == nullptr || k_ring == nullptr || v_ring == nullptr)
    return n == 0 ? RKV_OK : RKV_ERR_NULL;
  if (dtype != RKV_BF16) return RKV_ERR_DTYPE;
  if (n_kv_heads < 1 || (head_dim != 64 && head_dim != 128)) return RKV_ERR_SHAPE;
  if (pos_first < 0 || n < 0) return RKV_ERR_ARG;
  if (!aligned16(k_src, v_src, k_ring, v_ring)) return RKV_ERR_ARG;
  if (ring_size < kChunk || ring_size % kChunk != 0 || n > ring_size) return RKV_ERR_RING;
  rkv::ScatterArgs a{};
  a.k_src = static_cast<const uint16_t*>(k_src);
  a.v_src = static_cast<const uint16_t*>(v_src);
  a.pos_first = pos_first;
  a.n = n;
  a.n_kv_heads = n_kv_heads;
  a.head_dim = head_dim;
  a.k_dst = static_cast<uint16_t*>(k_ring);
  a.v_dst = static_cast<uint16_t*>(v_ring);
  a.pt = nullptr;
  a.n_slots = ring_size / kChunk;
  a.ring_size = ring_size;
  return hip_status(rkv::launch_scatter(a, static_cast<hipStream_t>(stream)));
}

int32_t ref_layout_to_paged(const void* k_src, const void* v_src, int64_t pos_first,
                            int64_t n, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                            void* k_pool, void* v_pool, const int32_t* page_table,
                            int32_t n_table, int32_t n_slots, int32_t chunk_size,
                            void* stream) {
  if (k_src == nullptr || v_src == nullptr || k_pool == nullptr || v_pool == nullptr ||
      page_table == nullptr)
    return n == 0 ? RKV_OK : RKV_ERR_NULL;
  if (dtype != RKV_BF16) return RKV_ERR_DTYPE;
  if (n_kv_heads < 1 || (head_dim != 64 && head_dim != 128)) return RKV_ERR_SHAPE;
  if (pos_first < 0 || n < 0) return RKV_ERR_ARG;
  if (!aligned16(k_src, v_src, k_pool, v_pool)) return RKV_ERR_ARG;
  if (chunk_size != kChunk || n_slots < 1) return RKV_ERR_TABLE;
  if (n > 0 && (pos_first + n - 1) / kChunk >= n_table) return RKV_ERR_TABLE;
  rkv::ScatterArgs a{};
  a.k_src = static_cast<const uint16_t*>(k_src);
  a.v_src = static_cast<const uint16_t*>(v_src);
  a.pos_first = pos_first;
  a.n = n;
  a.n_kv_heads = n_kv_heads;
  a.head_dim = head_dim;
  a.k_dst = static_cast<uint16_t*>(k_pool);
  a.v_dst = static_cast<uint16_t*>(v_pool);
  a.pt = page_table;
  a.n_table = n_table;
  a.n_slots = n_slots;
  a.ring_size = 0;
  return hip_status(rkv::launch_scatter(a, static_cast<hipStream_t>(stream)));
}

// ---- KV append of a verify block -------------------------------------------------------

int32_t verify_kv_append_ring(const void* k_new, const void* v_new, int32_t n,
                              int64_t pos_first, int32_t n_kv_heads, int32_t head_dim,
                              void* k_ring, void* v_ring, int32_t ring_size, void* stream) {
  if (k_new == nullptr || v_new == nullptr || k_ring == nullptr || v_ring == nullptr)
    return RKV_ERR_NULL;
  if (n_kv_heads < 1 || (head_dim != 64 && head_dim != 128)) return RKV_ERR_SHAPE;
  if (n < 1 || n > RKV_MAX_APPEND || pos_first < 0) return RKV_ERR_ARG;
  if (!aligned16(k_new, v_new, k_ring, v_ring)) return RKV_ERR_ARG;
  if (ring_size < kChunk || ring_size % kChunk != 0 || n > ring_size) return RKV_ERR_RING;
  rkv::ScatterArgs a{};
  a.k_src = static_cast<const uint16_t*>(k_new);
  a.v_src = static_cast<const uint16_t*>(v_new);
  a.pos_first = pos_first;
  a.n = n;
  a.n_kv_heads = n_kv_heads;
  a.head_dim = head_dim;
  a.k_dst = static_cast<uint16_t*>(k_ring);
  a.v_dst = static_cast<uint16_t*>(v_ring);
  a.pt = nullptr;
  a.n_slots = ring_size / kChunk;
  a.ring_size = ring_size;
  return hip_status(rkv::launch_scatter(a, static_cast<hipStream_t>(stream)));
}

int32_t verify_kv_append_ring_dev(const void* k_new, const void* v_new, int32_t n,
                                  const int64_t* d_pos, int64_t pos_cap, int32_t n_kv_heads,
                                  int32_t head_dim, void* k_ring, void* v_ring, int32_t ring_size,
                                  void* stream) {
  if (k_new == nullptr || v_new == nullptr || k_ring == nullptr || v_ring == nullptr ||
      d_pos == nullptr)
    return RKV_ERR_NULL;
  if (n_kv_heads < 1 || (head_dim != 64 && head_dim != 128)) return RKV_ERR_SHAPE;
  if (n < 1 || n > RKV_MAX_APPEND || pos_cap < 0) return RKV_ERR_ARG;
  if (!aligned16(k_new, v_new, k_ring, v_ring)) return RKV_ERR_ARG;
  if (ring_size < kChunk || ring_size % kChunk != 0 || n > ring_size) return RKV_ERR_RING;
  rkv::ScatterArgs a{};
  a.k_src = static_cast<const uint16_t*>(k_new);
  a.v_src = static_cast<const uint16_t*>(v_new);
  a.n = n;
  a.n_kv_heads = n_kv_heads;
  a.head_dim = head_dim;
  a.k_dst = static_cast<uint16_t*>(k_ring);
  a.v_dst = static_cast<uint16_t*>(v_ring);
  a.n_slots = ring_size / kChunk;
  a.ring_size = ring_size;
  a.d_pos = d_pos;
  a.pos_cap = pos_cap;
  return hip_status(rkv::launch_scatter(a, static_cast<hipStream_t>(stream)));
}

int32_t verify_kv_append_paged_dev(const void* k_new, const void* v_new, int32_t n,
                                   const int64_t* d_pos, int64_t pos_cap, int32_t n_kv_heads,
                                   int32_t head_dim, void* k_pool, void* v_pool,
                                   const int32_t* page_table, int32_t n_table, int32_t n_slots,
                                   void* stream) {
  if (k_new == nullptr || v_new == nullptr || k_pool == nullptr || v_pool == nullptr ||
      page_table == nullptr || d_pos == nullptr)
    return RKV_ERR_NULL;
  if (n_kv_heads < 1 || (head_dim != 64 && head_dim != 128)) return RKV_ERR_SHAPE;
  if (n < 1 || n > RKV_MAX_APPEND || pos_cap < 0) return RKV_ERR_ARG;
  if (!aligned16(k_new, v_new, k_pool, v_pool)) return RKV_ERR_ARG;
  if (n_slots < 1 || n_table < 1) return RKV_ERR_TABLE;
  if ((pos_cap + n + kChunk - 1) / kChunk > n_table) return RKV_ERR_TABLE;
  rkv::ScatterArgs a{};
  a.k_src = static_cast<const uint16_t*>(k_new);
  a.v_src = static_cast<const uint16_t*>(v_new);
  a.n = n;
  a.n_kv_heads = n_kv_heads;
  a.head_dim = head_dim;
  a.k_dst = static_cast<uint16_t*>(k_pool);
  a.v_dst = static_cast<uint16_t*>(v_pool);
  a.pt = page_table;
  a.n_table = n_table;
  a.n_slots = n_slots;
  a.d_pos = d_pos;
  a.pos_cap = pos_cap;
  return hip_status(rkv::launch_scatter(a, static_cast<hipStream_t>(stream)));
}

int32_t verify_pos_advance(int64_t* d_pos, const int32_t* accept_len, void* stream) {
  if (d_pos == nullptr || accept_len == nullptr) return RKV_ERR_NULL;
  rkv::AdvanceArgs a{d_pos, accept_len};
  return hip_status(rkv::launch_advance(a, static_cast<hipStream_t>(stream)));
}

int32_t verify_kv_append_paged(const void* k_new, const void* v_new, int32_t n,
                               int64_t ctx_len, int32_t n_kv_heads, int32_t head_dim,
                               void* k_pool, void* v_pool, int32_t* page_table,
                               int32_t n_table, int32_t n_slots, int32_t first_chunk,
                               int32_t n_new, const int32_t* new_slots, void* stream) {
  if (k_new == nullptr || v_new == nullptr || k_pool == nullptr || v_pool == nullptr ||
      page_table == nullptr || (n_new > 0 && new_slots == nullptr))
    return RKV_ERR_NULL;
  if (n_kv_heads < 1 || (head_dim != 64 && head_dim != 128)) return RKV_ERR_SHAPE;
  if (n < 1 || n > RKV_MAX_APPEND || ctx_len < 0) return RKV_ERR_ARG;
  if (!aligned16(k_new, v_new, k_pool, v_pool)) return RKV_ERR_ARG;
  if (n_slots < 1 || n_table < 1) return RKV_ERR_TABLE;
  const int64_t c0 = (ctx_len + kChunk - 1) / kChunk;
  const int64_t c1 = (ctx_len + n + kChunk - 1) / kChunk;
  if (c1 > n_table) return RKV_ERR_TABLE;
  if (first_chunk != c0 || n_new != c1 - c0 || n_new > RKV_MAX_APPEND_CHUNKS) return RKV_ERR_ARG;
  rkv::ScatterArgs a{};
  for (int32_t i = 0; i < n_new; ++i) {
    if (new_slots[i] < 0 || new_slots[i] >= n_slots) return RKV_ERR_TABLE;
    a.new_slots[i] = new_slots[i];
  }
  a.k_src = static_cast<const uint16_t*>(k_new);
  a.v_src = static_cast<const uint16_t*>(v_new);
  a.pos_first = ctx_len;
  a.n = n;
  a.n_kv_heads = n_kv_heads;
  a.head_dim = head_dim;
  a.k_dst = static_cast<uint16_t*>(k_pool);
  a.v_dst = static_cast<uint16_t*>(v_pool);
  a.pt = page_table;
  a.n_table = n_table;
  a.n_slots = n_slots;
  a.ring_size = 0;
  a.pt_w = page_table;
  a.first_new = first_chunk;
  a.n_new = n_new;
  return hip_status(rkv::launch_scatter(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
