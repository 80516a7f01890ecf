/*
 * ring_kv.h -- C interface of libring_kv, the speculative-decoding verify step on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (lucebox post "Laguna XS 2.1 33B on a RTX 3090: 296 tok/s peak, 152 tok/s
 * at 256K context"):
 *   - a drafter proposes a block of tokens that the target checks in one batched
 *     forward ("The model, fast MoE with a drafter in the box");
 *   - sliding-window layers attend a ring indexed by position, slot = pos mod 2048, window 512
 *     ("3. Ring caches for the sliding-window layers");
 *   - full-attention layers attend a GPU pool of 64-token chunks ("Three
 *     optimizations", item 1, KVFlash paging), found through a page table;
 *   - what is committed equals what greedy decoding by the target produces: the longest agreeing
 *     drafted prefix plus the target's next token ("TL;DR"; "The model, fast MoE with
 *     a drafter in the box").
 *
 * Conventions shared by every call
 * --------------------------------
 * Memory.  Every tensor pointer is a DEVICE pointer owned by the caller (the library
 *   never allocates, frees, or keeps a pointer after the call returns).  Scratch
 *   memory is passed in as `workspace`; query its size with the matching
 *   *_workspace_bytes() function.
 * Streams.  `stream` is a hipStream_t (NULL: the default stream).  Calls enqueue
 *   kernels and return without synchronising; the caller keeps every buffer alive
 *   until the stream has passed the work.
 * Errors.  Every call returns an rkv_status.  All shape, dtype, pointer and size
 *   checks run on the host before any HIP call, so a rejected call touches no
 *   device state.  A failed launch returns RKV_ERR_HIP; the launch status is the
 *   launch's own, so an error some earlier HIP call left in the thread's last-error
 *   state is neither reported nor cleared.  No C++ exception crosses this interface.
 * Device.  Split counts and row tiles follow the current device's compute-unit count
 *   (queried once per device); the workspace sizes depend on it, so size and call on
 *   the same device.
 * Determinism.  Identical inputs give bit-identical outputs: no float atomics, a
 *   fixed reduction order, and paged work ordered by logical chunk (never by
 *   physical slot), so permuting the pool changes nothing.
 *
 * Attention definition (every layout).  Query i of the block (0 <= i < q_len) sits at
 * absolute position p_i; query head h reads KV head g = h / G, G = n_q_heads /
 * n_kv_heads.  It attends keys j with lo_i <= j <= p_i, where lo_i = 0 (full
 * causal) or max(0, p_i - window + 1) (a window of `window` keys including its own
 * position).  With s_j = scale * <Q[i][h], K(j)[g]>:
 *     out[i][h][:] = sum_j exp(s_j - m) V(j)[g][:] / sum_j exp(s_j - m),  m = max_j s_j
 *     lse[i][h]    = m + ln sum_j exp(s_j - m)            (natural log)
 * Query i sees the block's earlier tokens and itself, so row i equals single-token
 * decoding at context p_i + 1.
 *
 * Layouts (row-major, innermost last)
 *   Q                 [q_len][n_q_heads][head_dim]           bf16 or f32
 *   contiguous K, V   [ctx_len][n_kv_heads][head_dim]        same dtype as Q
 *   chunked K store   [n_slots][n_kv_heads][64][head_dim]    bf16   (key-major chunk)
 *   chunked V store   [n_slots][n_kv_heads][head_dim][64]    bf16   (dimension-major chunk)
 *   out               [q_len][n_q_heads][head_dim]           f32
 *   lse               [q_len][n_q_heads]                     f32 (may be NULL)
 * A chunked store holds 64 consecutive positions per slot.  The paged pool puts
 * logical chunk c = j / 64 in slot page_table[c]; the ring is a store of
 * ring_size / 64 slots that puts position j at ring slot j mod ring_size, i.e. chunk
 * slot (j mod ring_size) / 64, offset j mod 64.  V is kept dimension-major inside a
 * chunk so that the PV product streams it without a transpose.
 */
#ifndef RING_KV_H
#define RING_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RKV_ABI_VERSION 1
#define RKV_CHUNK 64            /* positions per chunk slot */
/* Rows per KV head, q_len * (n_q_heads / n_kv_heads), that one call may carry.  A verify block
 * (16 drafts: 64 rows at G = 4) and a batched prefill block (lucebox post, "TL;DR": prefill
 * as pooled batches plus ring attention; 1024 tokens: 4096 rows at G = 4) go through the same
 * calls.  Up to 256 rows the chunked calls stream the KV with 16-, 32- or 64-row tiles; longer
 * blocks run a matrix-core kernel with 64-, 128- or 256-row tiles.  Same definition, layouts and
 * results. */
#define RKV_MAX_ROWS 16384

typedef enum rkv_status {
  RKV_OK = 0,
  RKV_ERR_NULL = -1,        /* a required pointer is NULL */
  RKV_ERR_SHAPE = -2,       /* head counts, head_dim, q_len or ctx_len out of range */
  RKV_ERR_DTYPE = -3,       /* dtype not supported by this call */
  RKV_ERR_RING = -4,        /* ring too small for window + block, ring_size not a multiple of
                               64, or ring_head is not pos0 mod ring_size */
  RKV_ERR_TABLE = -5,       /* chunk_size is not 64, or the page table / pool is too small */
  RKV_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than *_workspace_bytes() */
  RKV_ERR_HIP = -7,         /* a HIP launch failed */
  RKV_ERR_ARG = -8          /* another argument out of range (window, splits, sizes) */
} rkv_status;

typedef enum rkv_dtype { RKV_F32 = 0, RKV_BF16 = 1 } rkv_dtype;

typedef struct rkv_attn_dims {
  int32_t q_len;        /* queries in the verify block, >= 1 (16 for a 16-token draft) */
  int32_t n_q_heads;    /* Hq, a multiple of n_kv_heads */
  int32_t n_kv_heads;   /* Hkv >= 1 */
  int32_t head_dim;     /* 64 or 128 */
  float scale;          /* softmax scale; 0 selects 1/sqrt(head_dim) */
  int32_t dtype;        /* rkv_dtype of Q, K and V */
} rkv_attn_dims;

int32_t rkv_abi_version(void);
const char* rkv_status_str(int32_t status);

/* ---------------------------------------------------------------------------------
 * Contiguous reference layout (GPU-side reference for the chunked calls, and plain
 * decode with q_len = 1).  The post verifies the whole drafted block in one batched
 * forward whose result must equal decoding the tokens one at a time (lucebox post, "The
 * model, fast MoE with a drafter in the box"); this call computes that batched attention
 * over rows stored in plain position order, so row i of a block equals the q_len = 1
 * call at context ctx_len - q_len + i + 1.  Keys are positions 0 .. ctx_len-1 in k, v
 * [ctx_len][Hkv][D] (row-major, caller-owned device memory); query i sits at
 * ctx_len - q_len + i.  window = 0: full causal, window > 0: sliding window of that
 * many keys (the window layers' 512, "3. Ring caches for the sliding-window layers").
 * dtype f32 or bf16; every arithmetic step runs in f32.  num_splits = 0 picks a split
 * of the key range; any value gives the same result up to f32 rounding.  Workspace:
 * decode_attn_ref_layout_workspace_bytes() bytes (0: none needed, NULL allowed).
 * Status: RKV_ERR_NULL (q, k, v, out), RKV_ERR_SHAPE (dims, ctx_len < q_len),
 * RKV_ERR_ARG (window or num_splits < 0), RKV_ERR_WORKSPACE, RKV_ERR_HIP.
 * ------------------------------------------------------------------------------- */
size_t decode_attn_ref_layout_workspace_bytes(const rkv_attn_dims* dims, int64_t ctx_len,
                                              int32_t num_splits);
int32_t decode_attn_ref_layout(const rkv_attn_dims* dims, const void* q, const void* k,
                               const void* v, int64_t ctx_len, int32_t window,
                               int32_t num_splits, void* workspace, size_t workspace_bytes,
                               float* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------------
 * Sliding-window verify attention over a position ring (lucebox post, "3. Ring caches
 * for the sliding-window layers": the window layers read a ring of their own, slot = pos
 * mod 2048, instead of the paged pool).
 *   pos0       absolute position of query 0; query i sits at pos0 + i
 *   ring_head  the slot of query 0; must equal pos0 mod ring_size (checked)
 *   ring_size  positions the ring holds, a multiple of 64, >= window + q_len - 1
 *   window     keys per query including its own position, >= 1
 * The ring must hold positions max(0, pos0+q_len-ring_size) .. pos0+q_len-1, the
 * block's own rows included.  k_ring [ring_size/64][Hkv][64][D], v_ring
 * [ring_size/64][Hkv][D][64], bf16; Q bf16.  Slots holding no position may contain
 * anything (they are masked and never multiply a result).
 * The span of the window is split into num_splits ranges of whole chunks (0: one chunk
 * per range, every chunk in flight at once, for a verify block; a block of more than 256
 * rows per KV head is not split, its row tiles fill the chip) whose partials a
 * log-sum-exp merge combines.
 * One range spans at most 2^22 chunks (RKV_ERR_SHAPE otherwise).
 * Workspace (caller-owned device memory, needed when the span is split): a workspace of at
 * least verify_attn_ring_workspace_bytes() bytes starts with RKV_RING_COUNTER_BYTES of
 * counters, which must be zero before the workspace's first use and which every call leaves
 * ready for the next (each 128-byte group line: an arrival count, returned to zero, and a
 * generation word that moves by one per call); with them the call merges the partials inside
 * its one launch where it can (the
 * workgroups of each KV head and row tile, all on one XCD, wait for each other's partials and
 * each merges a share of the tile's rows; used when the grid fits one workgroup per compute
 * unit).  Calls that share a workspace must not overlap, and the counters must not be written
 * by anything else.  A smaller workspace that still holds the call's partials works without
 * counters: the partials are merged by a second launch, with the same result bits.
 * ------------------------------------------------------------------------------- */
#define RKV_RING_COUNTER_BYTES 8192
size_t verify_attn_ring_workspace_bytes(const rkv_attn_dims* dims, int32_t ring_size,
                                        int32_t window, int32_t num_splits);
int32_t verify_attn_ring(const rkv_attn_dims* dims, const void* q, const void* k_ring,
                         const void* v_ring, int64_t pos0, int32_t ring_head,
                         int32_t ring_size, int32_t window, int32_t num_splits,
                         void* workspace, size_t workspace_bytes, float* out, float* lse,
                         void* stream);

/* ---------------------------------------------------------------------------------
 * Full-attention verify attention over the paged pool of 64-token chunks (lucebox
 * post, "Three optimizations", item 1).  Keys are positions 0 .. ctx_len-1; query i
 * sits at ctx_len - q_len + i (ctx_len counts the block).  Logical chunk c lives in
 * pool slot page_table[c] (device int32 array of n_table >= ceil(ctx_len/64)
 * entries); k_pool [n_slots][Hkv][64][D], v_pool [n_slots][Hkv][D][64], bf16; Q
 * bf16.  chunk_size must be 64.  Positions >= ctx_len in the last chunk may hold
 * anything.  An entry outside [0, n_slots) is never dereferenced: its chunk
 * contributes nothing (a contract breach, not an error the call can report).
 *
 * The key range is split into num_splits ranges of whole chunks (0: chosen from the
 * context and the device's compute units, 256 on MI355X); each range yields a partial result
 * and a log-sum-exp merge combines them.  Any split gives the same result up to
 * rounding: the bf16 weights of the PV product are rounded against each range's own
 * running maximum, so split counts differ by about 1e-4 on N(0,1) inputs (within the
 * bf16 tolerance of the exact result either way).  One split spans at most 2^22 chunks (RKV_ERR_SHAPE otherwise):
 * with num_splits = 1 that bounds ctx_len by 2^28.
 * ------------------------------------------------------------------------------- */
size_t verify_attn_paged_workspace_bytes(const rkv_attn_dims* dims, int64_t ctx_len,
                                         int32_t chunk_size, int32_t num_splits);
int32_t verify_attn_paged(const rkv_attn_dims* dims, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* page_table, int32_t n_table,
                          int32_t n_slots, int32_t chunk_size, int64_t ctx_len,
                          int32_t num_splits, void* workspace, size_t workspace_bytes,
                          float* out, float* lse, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): verify_attn_paged with no workspace argument.  The
 * split partials go to a static device array inside the library, RKV_NOALLOC_SCRATCH_BYTES
 * (16 MiB) per device, held from the first call on a device until the process ends; the call
 * itself allocates nothing.  Same arguments (minus the workspace), kernels, splits and results
 * as verify_attn_paged.  RKV_ERR_WORKSPACE when the call's partials,
 * verify_attn_paged_workspace_bytes(dims, ctx_len, 64, num_splits) bytes, exceed the array
 * (4 KV heads x 64 splits x 64 rows fit: every verify block of the named workloads; a
 * 1,024-token prefill block does not); RKV_ERR_HIP if the array's address cannot be found.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on different
 * streams, or from different threads) race on it; calls ordered on one stream do not. */
#define RKV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int32_t verify_attn_paged_noalloc(const rkv_attn_dims* dims, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* page_table, int32_t n_table,
                                  int32_t n_slots, int32_t chunk_size, int64_t ctx_len,
                                  int32_t num_splits, float* out, float* lse, void* stream);

/* Split count verify_attn_paged uses for num_splits = 0 (host-only, no HIP call). */
int32_t verify_attn_paged_auto_splits(const rkv_attn_dims* dims, int64_t ctx_len,
                                      int32_t chunk_size);

/* ---------------------------------------------------------------------------------
 * The paged call in two phases, for callers that time or distribute them (partials
 * of disjoint key ranges, e.g. computed on different devices, merge the same way).
 * Split s covers logical chunks [s*cps, min((s+1)*cps, n_chunks)) with n_chunks =
 * ceil(ctx_len/64), cps = ceil(n_chunks/num_splits); num_splits >= 1 here, and
 * cps <= 2^22 (RKV_ERR_SHAPE otherwise).
 *   part_out  [n_kv_heads][num_splits][q_len*G][D] f32: the split's normalised output
 *   part_lse  [n_kv_heads][num_splits][q_len*G]    f32: natural-log lse over the split's
 *             keys, -inf where a row sees no key of the split (then part_out row = 0)
 * Row r of a KV head is query r / G, query head g*G + r % G.
 * ------------------------------------------------------------------------------- */
int32_t verify_attn_paged_partial(const rkv_attn_dims* dims, const void* q,
                                  const void* k_pool, const void* v_pool,
                                  const int32_t* page_table, int32_t n_table, int32_t n_slots,
                                  int32_t chunk_size, int64_t ctx_len, int32_t num_splits,
                                  float* part_out, float* part_lse, void* stream);

/* Log-sum-exp merge of num_splits partials laid out as above:
 *   M = max_s lse_s, w_s = exp(lse_s - M), out = sum_s w_s O_s / sum_s w_s,
 *   lse = M + ln sum_s w_s   (splits with lse_s = -inf carry no weight).
 * dims->dtype is ignored.  out [q_len][Hq][D] f32, lse [q_len][Hq] f32 or NULL. */
int32_t attn_merge_partials(const rkv_attn_dims* dims, int32_t num_splits,
                            const float* part_out, const float* part_lse, float* out,
                            float* lse, void* stream);

/* ---------------------------------------------------------------------------------
 * Greedy acceptance (lucebox post, "TL;DR" and "The model, fast MoE with a drafter in
 * the box": verify-exact speculative decoding, exact greedy equivalence).
 *   logits     [n_draft+1][vocab] f32, finite; row r is the target's distribution
 *              after the committed prefix and drafts 0..r-1
 *   proposals  [n_draft] int32 drafted tokens
 * t_r = the first index of the maximum of row r (float32 compare, -0 == +0);
 * a = the first r < n_draft with t_r != proposals[r], else n_draft.
 *   accept_len [1] int32 <- a
 *   committed  [n_draft+1] int32 <- proposals[0..a) then t_a; entries after a are -1
 *   row_argmax [n_draft+1] int32 <- t_r (may be NULL)
 * 0 <= n_draft <= 255, vocab >= 1.  NaN logits give an unspecified (but in-range)
 * result.  Calls sharing a workspace must not overlap.
 * ------------------------------------------------------------------------------- */
size_t verify_accept_workspace_bytes(int32_t n_draft, int32_t vocab);
int32_t verify_accept(const float* logits, int32_t n_draft, int32_t vocab,
                      const int32_t* proposals, int32_t* accept_len, int32_t* committed,
                      int32_t* row_argmax, void* workspace, size_t workspace_bytes,
                      void* stream);

/* ---------------------------------------------------------------------------------
 * Layout helpers: copy n contiguous rows k_src, v_src [n][Hkv][D] holding positions
 * pos_first .. pos_first+n-1 into a ring or into the paged pool, K key-major and V
 * dimension-major per chunk.  The ring puts position p at slot p mod ring_size (lucebox
 * post, "3. Ring caches for the sliding-window layers": slot = pos mod 2048); the pool
 * puts it in chunk p / 64 at offset p mod 64, the chunk living in slot page_table[p/64]
 * ("Three optimizations", item 1: 64-token chunks).  This is also how a verify block's
 * own rows are appended before attention.  All pointers are caller-owned device memory,
 * 16-byte aligned (RKV_ERR_ARG otherwise); dtype must be bf16.  For the ring, n <= ring_size (RKV_ERR_RING otherwise); for the
 * pool, the table must cover the last position (RKV_ERR_TABLE).  Pool entries outside
 * [0, n_slots) are skipped on the device.  n = 0 does nothing.
 * ------------------------------------------------------------------------------- */
int32_t ref_layout_to_ring(const void* k_src, const void* v_src, int64_t pos_first, int64_t n,
                           int32_t n_kv_heads, int32_t head_dim, int32_t dtype, void* k_ring,
                           void* v_ring, int32_t ring_size, void* stream);
int32_t ref_layout_to_paged(const void* k_src, const void* v_src, int64_t pos_first,
                            int64_t n, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                            void* k_pool, void* v_pool, const int32_t* page_table,
                            int32_t n_table, int32_t n_slots, int32_t chunk_size,
                            void* stream);

/* ---------------------------------------------------------------------------------
 * KV append and rollback for the verify block.  Before verify attention the block's own
 * n K/V rows (positions ctx .. ctx+n-1) join the stores; after the accept, the a+1 kept
 * rows are committed and the rest are left to be overwritten (lucebox post, "3. Ring
 * caches for the sliding-window layers": slot = pos mod 2048; "Three optimizations",
 * item 1: a pool of 64-token chunks located through a page table; the verify step keeps
 * exactly what greedy decoding by the target would produce).
 *
 * Rows and stores are 16-byte aligned device memory (RKV_ERR_ARG otherwise).
 * Ring: verify_kv_append_ring writes row i (position pos_first+i) at ring slot
 * (pos_first+i) mod ring_size, 1 <= n <= RKV_MAX_APPEND, n <= ring_size.  Rolling back
 * needs no call: a rejected position is written again by the next block's append before
 * any attention reads it.
 *
 * Pool: a host-side pager owns the free list of pool slots and a host copy of the page
 * table; ctx is its committed length.
 *   rkv_pager_reserve(p, n, &first_chunk, &n_new, slots)  allocates slots for the chunks
 *       that positions ctx .. ctx+n-1 start: chunks first_chunk .. first_chunk+n_new-1
 *       (first_chunk = ceil(ctx/64)) get slots[0 .. n_new-1] (capacity
 *       RKV_MAX_APPEND_CHUNKS).  One block may be pending at a time.
 *   verify_kv_append_paged(...)  writes those table entries into the device page table and
 *       the n rows into the pool, in one launch (positions in chunks below first_chunk use
 *       the device table's existing entries).
 *   rkv_pager_commit(p, n_keep)  the first n_keep rows of the pending block are committed
 *       (ctx += n_keep, 0 <= n_keep <= n); its chunks that hold no committed position go
 *       back to the free list, and their host table entries become -1.
 * Slots come from a stack that starts as 0, 1, 2, ...; freed slots are reused first, the
 * most recently freed one first.  Status: RKV_ERR_TABLE when the free list or the table
 * cannot cover the block (nothing changes), RKV_ERR_ARG for a reserve while a block is
 * pending, a commit without one, n out of range or n_keep > n, RKV_ERR_NULL for null
 * pointers.  A pager is host memory only and not thread-safe; destroy it with
 * rkv_pager_destroy.
 * ------------------------------------------------------------------------------- */
#define RKV_MAX_APPEND 1024
#define RKV_MAX_APPEND_CHUNKS 17        /* a block of 1024 rows starts at most 17 chunks */

typedef struct rkv_pager rkv_pager;
rkv_pager* rkv_pager_create(int32_t n_slots, int32_t n_table);   /* NULL on sizes < 1 */
void rkv_pager_destroy(rkv_pager* p);
int64_t rkv_pager_ctx_len(const rkv_pager* p);                    /* -1 for NULL */
int32_t rkv_pager_free_slots(const rkv_pager* p);                 /* -1 for NULL */
/* host copy of table entries 0 .. n-1 into out (-1: no slot, RKV_PAGED_OUT: on the host);
 * n <= n_table */
int32_t rkv_pager_table(const rkv_pager* p, int32_t* out, int32_t n);
int32_t rkv_pager_reserve(rkv_pager* p, int32_t n, int32_t* first_chunk, int32_t* n_new,
                          int32_t* slots);
int32_t rkv_pager_commit(rkv_pager* p, int32_t n_keep);

/* k_new, v_new [n][Hkv][D] bf16 (device), the rows of positions pos_first .. */
int32_t verify_kv_append_ring(const void* k_new, const void* v_new, int32_t n,
                              int64_t pos_first, int32_t n_kv_heads, int32_t head_dim,
                              void* k_ring, void* v_ring, int32_t ring_size, void* stream);
/* rows of positions ctx_len .. ctx_len+n-1; first_chunk must be ceil(ctx_len/64) and n_new
 * the number of chunks the block starts (as rkv_pager_reserve reports them); new_slots is a
 * host array of n_new slots in [0, n_slots); page_table is the device table (written for the
 * new chunks).  RKV_ERR_TABLE if the block does not fit the table or the slots are out of
 * range. */
int32_t verify_kv_append_paged(const void* k_new, const void* v_new, int32_t n,
                               int64_t ctx_len, int32_t n_kv_heads, int32_t head_dim,
                               void* k_pool, void* v_pool, int32_t* page_table,
                               int32_t n_table, int32_t n_slots, int32_t first_chunk,
                               int32_t n_new, const int32_t* new_slots, void* stream);

/* ---------------------------------------------------------------------------------
 * One captured step replayed across decode steps (lucebox post, "The model, fast MoE with a
 * drafter in the box": the decode loop is fused and replayed as a graph; "Three
 * optimizations", item 1: prefill blocks are graph replays too).  A captured HIP graph
 * replays the kernel arguments it recorded, so a step whose positions are arguments can
 * only be replayed at the same positions.  These calls read the block's position from
 * device memory instead:
 *   d_pos   device int64: the absolute position of the block's first row, which is the
 *           committed length of the sequence (query i and appended row i sit at *d_pos + i;
 *           the pool's context is *d_pos + q_len)
 *   pos_cap the largest value *d_pos may take while the graph is replayed; the split layout
 *           (and the workspace) cover every position up to it
 * and verify_pos_advance moves *d_pos past the tokens a step committed, on the device:
 *   *d_pos += *accept_len + 1     (the a accepted drafts and the target's next token)
 * so that append -> attention -> accept -> advance, captured once, is the decode loop.
 * The pool calls read the slot of every chunk from page_table: the caller reserves the
 * slots of every chunk the positions up to pos_cap + n can reach before capturing (there
 * is no allocation inside a replay).  A device value outside [0, pos_cap] makes the
 * attention calls write NaN to out and lse and the append calls write nothing.  Same
 * definition, layouts and results as verify_attn_ring / verify_attn_paged /
 * verify_kv_append_* at the position *d_pos holds when the stream runs the call; verify
 * blocks only (q_len * G <= 256, RKV_ERR_SHAPE otherwise).
 *   ring workspace: verify_attn_ring_workspace_bytes(dims, ring_size, window, num_splits)
 *   pool workspace: verify_attn_paged_workspace_bytes(dims, pos_cap + q_len, 64, num_splits)
 * Status as the position-argument calls, plus RKV_ERR_NULL for d_pos and RKV_ERR_ARG for
 * pos_cap < 0; the pool calls return RKV_ERR_TABLE when the table cannot hold position
 * pos_cap + q_len - 1 (attention) or pos_cap + n - 1 (append).
 * ------------------------------------------------------------------------------- */
int32_t verify_attn_ring_dev(const rkv_attn_dims* dims, const void* q, const void* k_ring,
                             const void* v_ring, const int64_t* d_pos, int64_t pos_cap,
                             int32_t ring_size, int32_t window, int32_t num_splits,
                             void* workspace, size_t workspace_bytes, float* out, float* lse,
                             void* stream);
int32_t verify_attn_paged_dev(const rkv_attn_dims* dims, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* page_table, int32_t n_table,
                              int32_t n_slots, int32_t chunk_size, const int64_t* d_pos,
                              int64_t pos_cap, int32_t num_splits, void* workspace,
                              size_t workspace_bytes, float* out, float* lse, void* stream);
int32_t verify_kv_append_ring_dev(const void* k_new, const void* v_new, int32_t n,
                                  const int64_t* d_pos, int64_t pos_cap, int32_t n_kv_heads,
                                  int32_t head_dim, void* k_ring, void* v_ring, int32_t ring_size,
                                  void* stream);
int32_t verify_kv_append_paged_dev(const void* k_new, const void* v_new, int32_t n,
                                   const int64_t* d_pos, int64_t pos_cap, int32_t n_kv_heads,
                                   int32_t head_dim, void* k_pool, void* v_pool,
                                   const int32_t* page_table, int32_t n_table, int32_t n_slots,
                                   void* stream);
int32_t verify_pos_advance(int64_t* d_pos, const int32_t* accept_len, void* stream);

/* ---------------------------------------------------------------------------------
 * The block's append and its attention in one launch (the decode loop's two calls per layer,
 * verify_kv_append_*_dev then verify_attn_*_dev, as one): k_new, v_new [q_len][Hkv][D] bf16 are
 * the block's own rows for positions *d_pos .. *d_pos + q_len - 1 (the block's inputs: the last
 * committed token and the drafts); they are written into their ring or pool slots and attended,
 * with the same results and the same store contents as the two calls.  Arguments, workspace and
 * status as verify_attn_ring_dev / verify_attn_paged_dev, plus RKV_ERR_NULL for k_new or v_new
 * and RKV_ERR_ARG for a row or store pointer that is not 16-byte aligned.  The pool's table
 * must hold the slots of the block's chunks (reserved before capture); a position outside
 * [0, pos_cap] writes nothing and gives NaN attention.
 * ------------------------------------------------------------------------------- */
int32_t verify_attn_ring_append_dev(const rkv_attn_dims* dims, const void* q, const void* k_new,
                                    const void* v_new, void* k_ring, void* v_ring,
                                    const int64_t* d_pos, int64_t pos_cap, int32_t ring_size,
                                    int32_t window, int32_t num_splits, void* workspace,
                                    size_t workspace_bytes, float* out, float* lse, void* stream);
int32_t verify_attn_paged_append_dev(const rkv_attn_dims* dims, const void* q, const void* k_new,
                                     const void* v_new, void* k_pool, void* v_pool,
                                     const int32_t* page_table, int32_t n_table, int32_t n_slots,
                                     int32_t chunk_size, const int64_t* d_pos, int64_t pos_cap,
                                     int32_t num_splits, void* workspace, size_t workspace_bytes,
                                     float* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------------
 * Host paging of the pool (lucebox post, "Three optimizations", item 1: only part of the
 * context stays in the GPU pool and 64-token chunks move to host memory and back without any
 * change to their bits; the drafter scores which chunks stay, outside this library).
 *
 * Host chunk store: k_host [n_host][Hkv][64][D], v_host [n_host][Hkv][D][64] bf16 in host
 * memory, one entry per logical chunk (entry c holds chunk c), laid out like a pool slot.
 * Allocate it pinned (hipHostMalloc) so that the copies run asynchronously; pageable memory
 * works, but the copies then wait for the host.
 *   kv_page_out  pool slot slots[i] -> host entry chunk_ids[i], i < n (K and V, bit-exact)
 *   kv_page_in   host entry chunk_ids[i] -> pool slot slots[i]
 * slots and chunk_ids are host arrays, read before the call returns; chunk ids must be
 * distinct in a page-out and slots distinct in a page-in.  RKV_PAGE_BATCH chunks at a time
 * cross PCIe one of two ways: when the host store is pinned memory the device can address, a
 * kernel copies each chunk straight between its slot and its host entry (every page-out, and
 * page-ins of scattered chunk ids); otherwise a kernel packs the chunks into a device
 * workspace and the copy engines move one copy per run of consecutive chunk ids.  Pass a
 * workspace of kv_page_workspace_bytes(n_kv_heads, head_dim, n) bytes either way.  Both
 * calls are asynchronous on `stream`: the host entries (page-out) or the slots (page-in) hold
 * the data once the stream has passed the call, and a slot freed by a page-out may be
 * rewritten by any later work on that stream.
 * Status: RKV_ERR_NULL; RKV_ERR_SHAPE (head counts, head_dim); RKV_ERR_ARG (n < 0, a chunk id
 * outside [0, n_host), a repeated chunk id or slot); RKV_ERR_TABLE (a slot outside
 * [0, n_slots)); RKV_ERR_WORKSPACE; RKV_ERR_HIP.
 * ------------------------------------------------------------------------------- */
#define RKV_PAGE_BATCH 256
size_t kv_page_workspace_bytes(int32_t n_kv_heads, int32_t head_dim, int32_t n);
int32_t kv_page_out(const void* k_pool, const void* v_pool, int32_t n_kv_heads,
                    int32_t head_dim, int32_t n_slots, const int32_t* slots,
                    const int32_t* chunk_ids, int32_t n, void* k_host, void* v_host,
                    int64_t n_host, void* workspace, size_t workspace_bytes, void* stream);
int32_t kv_page_in(const void* k_host, const void* v_host, int64_t n_host,
                   const int32_t* chunk_ids, const int32_t* slots, int32_t n, void* k_pool,
                   void* v_pool, int32_t n_kv_heads, int32_t head_dim, int32_t n_slots,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Full-attention attention of a block (verify or prefill) over the resident subset of the
 * pool: the keys are the positions of the chunks listed in chunk_ids (host array, strictly
 * increasing, n_res >= 1 entries); chunk chunk_ids[i] is read from pool slot d_slots[i]
 * (device array).  Query i sits at ctx_len - q_len + i and sees the listed keys at or before
 * its position.  The chunks holding the block's positions (ctx_len-q_len .. ctx_len-1) must be
 * listed, as the last entries (RKV_ERR_TABLE otherwise); positions >= ctx_len in the last
 * chunk may hold anything.  Every earlier listed chunk is then wholly visible to every query,
 * so the call runs the paged kernels with d_slots as the table at the context
 * ctx_len - 64 * (chunks missing before the block's first chunk), n_res chunks long.  Splits
 * and outputs: as verify_attn_paged over n_res chunks; the workspace is
 * verify_attn_paged_workspace_bytes(dims, 64 * n_res, 64, num_splits) bytes. */
int32_t verify_attn_paged_resident(const rkv_attn_dims* dims, const void* q,
                                   const void* k_pool, const void* v_pool,
                                   const int32_t* d_slots, const int32_t* chunk_ids,
                                   int32_t n_res, int32_t n_slots, int64_t ctx_len,
                                   int32_t num_splits, void* workspace, size_t workspace_bytes,
                                   float* out, float* lse, void* stream);

/* The pager's side of host paging.  A chunk paged out has the table entry RKV_PAGED_OUT.
 *   rkv_pager_evict    n whole committed chunks (chunk < floor(ctx/64)) that have a slot: their
 *                      slots are written to slots[] (copy them out with kv_page_out before any
 *                      reuse) and return to the free list in the order given.
 *   rkv_pager_restore  n paged-out chunks each get the next free slot (slots[] out; copy the
 *                      data in with kv_page_in).
 *   rkv_pager_resident the chunks that have a slot (the pending block's included), in
 *                      increasing order: returns how many; writes up to cap of them to
 *                      chunk_ids and slots (both may be NULL when cap is 0).
 * All or nothing: RKV_ERR_ARG for a chunk that does not qualify or is repeated, RKV_ERR_TABLE
 * when the free list is too short for a restore, RKV_ERR_NULL for null pointers. */
#define RKV_PAGED_OUT (-2)
int32_t rkv_pager_evict(rkv_pager* p, const int32_t* chunk_ids, int32_t n, int32_t* slots);
int32_t rkv_pager_restore(rkv_pager* p, const int32_t* chunk_ids, int32_t n, int32_t* slots);
int32_t rkv_pager_resident(const rkv_pager* p, int32_t* chunk_ids, int32_t* slots, int32_t cap);

#ifdef __cplusplus
}
#endif

#endif /* RING_KV_H */
