// Internal launch interface between the C entry points (abi.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ring_kv.h"

namespace rkv {

// Compute units of the current device (hipDeviceAttributeMultiprocessorCount), queried once per
// device and cached; 256 (a whole MI355X) where the query fails, e.g. on a machine without a GPU.
int device_cu_count();

// Launch a kernel that takes one argument struct by value.  hipLaunchKernel returns the status of
// this launch alone; the thread's last-error state (which may hold an error of some earlier,
// unrelated HIP call) is neither read nor cleared.
template <typename A>
inline hipError_t launch_kernel(void (*fn)(A), dim3 grid, dim3 block, const A& a,
                                hipStream_t stream) {
  void* args[] = {const_cast<A*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), grid, block, args, 0, stream);
}

// Most chunks one split may span: positions inside a workgroup are 32-bit offsets from its
// split's first key.
constexpr int64_t kMaxSplitChunks = int64_t(1) << 22;

// Attention of one verify block over a chunked KV store (paged pool or position ring),
// split over ranges of whole chunks.  Rows of a KV head: r = i * G + (h - g * G).
struct ChunkAttnArgs {
  const uint16_t* q;      // [q_len][Hq][D] bf16
  const uint16_t* k;      // [n_slots][Hkv][64][D] bf16
  const uint16_t* v;      // [n_slots][Hkv][D][64] bf16
  const int32_t* pt;      // page table; nullptr selects the ring (slot = c mod n_slots)
  int32_t n_slots;        // pool slots, or ring chunk slots
  int32_t q_len, G, n_q_heads, n_kv_heads, head_dim;
  int64_t p0;             // position of query 0
  int32_t window;         // 0: full causal
  int64_t valid_lo;       // the store holds positions [valid_lo, valid_hi)
  int64_t valid_hi;
  int64_t c_first;        // first logical chunk of split 0
  int64_t n_chunks;       // logical chunks covered by all splits
  int32_t cps;            // chunks per split
  int32_t num_splits;
  float scale_log2;       // softmax scale * log2(e)
  float* out;             // part_o == nullptr: final output [q_len][Hq][D]
  float* lse;             //                    and lse [q_len][Hq] (may be nullptr)
  float* part_o;          // otherwise partials [Hkv][S][rows][D]
  float* part_lse;        //                    and [Hkv][S][rows]
  // Device-resident position (nullptr: p0 .. n_chunks above hold).  The block's first row sits
  // at *d_pos; p0, valid_lo, valid_hi, c_first and n_chunks are derived from it on the device
  // (pool: context *d_pos + q_len; ring: window span and stored range around it).  A value
  // outside [0, pos_cap] gives NaN outputs; num_splits * cps covers every value up to pos_cap.
  const int64_t* d_pos;
  int64_t pos_cap;
  int32_t ring_size;      // positions the ring holds (ring only)
  int32_t fill_wgs;       // workgroups of one round over the device (its compute units)
  // Counters of the one-launch ring layer (nullptr: the partials are merged by a second
  // launch): a 128-byte line per (KV head, row tile) holding an arrival counter (zero before
  // the launch and left zero by it) and a generation word (any value).
  int32_t* tickets;
  // The block's own K/V rows (nullptr: the store already holds them), [q_len][Hkv][D] bf16 for
  // positions p0 .. p0 + q_len - 1: written into their slots of the store (k_w, v_w: the same
  // memory as k, v) before they are read, so that the append and the attention are one launch.
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_w;
  uint16_t* v_w;
};

// Blocks of up to kVerifyMaxRows rows per KV head (a verify block: q_len * G) run the
// HBM-streaming kernel with 16-, 32- or 64-row tiles (the smallest whose grid fits one round of
// fill_wgs workgroups, one per compute unit); longer blocks (batched prefill) run the
// matrix-core kernel with tiles of kPrefillTileRows rows.  launch_chunk_attn picks the kernel.
constexpr int kVerifyMaxRows = 256;
constexpr int kPrefillTileRows = 256;
// The one-launch ring layer: the workgroups of one (KV head, row tile) all run on one XCD; once
// all of them have stored their partials, each merges a share of the tile's rows, reading the
// partials through that XCD's L2.  Used for ring splits up to kFuseMaxSplits whose (head, tile)
// groups divide evenly over the kXcds XCDs and whose grid fits one workgroup per compute unit.
constexpr int kFuseMaxSplits = 12;
constexpr int kXcds = 8;
// Bytes of counters the one-launch ring layer keeps at the start of a ring call's workspace: one
// kTicketStride-byte line per (KV head, row tile), holding the group's arrival counter and its
// generation word (the lines of different groups never share a cache line: every workgroup's
// add goes to the device-wide coherence point, and adds to one line queue there), for up to 64
// groups.
constexpr size_t kTicketBytes = RKV_RING_COUNTER_BYTES;
constexpr int kTicketStride = 128;
// Row tile of the prefill kernel: kPrefillTileRows, or half of it (two waves per row group, one
// per half of each chunk's keys) when the full tiles would leave most of the chip without a
// workgroup (fewer than `fill`, the compute units), or a quarter of it (two row groups) where
// even that grid of quarter tiles fits one round of `fill` workgroups (a block over the ring).
inline int prefill_tile_rows(int rows, int n_kv_heads, int num_splits, int fill) {
  auto grid = [&](int tile) {
    return (int64_t)n_kv_heads * num_splits * ((rows + tile - 1) / tile);
  };
  if (grid(kPrefillTileRows) >= fill) return kPrefillTileRows;
  if (grid(kPrefillTileRows / 4) <= fill) return kPrefillTileRows / 4;
  return kPrefillTileRows / 2;
}
// *merged: true when the launch also merged the partials into out / lse (the one-launch ring
// layer), so that no merge launch follows.
hipError_t launch_chunk_attn(const ChunkAttnArgs& a, hipStream_t stream, bool* merged);
hipError_t launch_prefill_attn(const ChunkAttnArgs& a, hipStream_t stream);

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  float* out;
  float* lse;
  int32_t q_len, G, n_q_heads, n_kv_heads, head_dim, num_splits;
};
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

// Contiguous-layout attention (f32 arithmetic), same partial format as above.
struct ContigArgs {
  const void* q;          // [q_len][Hq][D]
  const void* k;          // [ctx][Hkv][D]
  const void* v;
  int32_t dtype;          // 0 f32, 1 bf16
  int32_t q_len, G, n_q_heads, n_kv_heads, head_dim;
  int64_t ctx_len;
  int32_t window;
  int64_t c_first;        // first 64-key tile of split 0 (tiles below every window are skipped)
  int64_t n_chunks;       // tiles covered by all splits
  int32_t cps;
  int32_t num_splits;
  float scale_log2;
  float* out;
  float* lse;
  float* part_o;
  float* part_lse;
};
hipError_t launch_contig_attn(const ContigArgs& a, hipStream_t stream);

struct AcceptArgs {
  const float* logits;
  int32_t n_rows;         // n_draft + 1
  int32_t vocab;
  const int32_t* proposals;
  int32_t* accept_len;
  int32_t* committed;
  int32_t* row_argmax;    // may be nullptr
  float* part_val;        // [n_rows][parts]
  int32_t* part_idx;      // [n_rows][parts]
  int32_t parts;
  int32_t part_len;
};
hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream);

// *pos += *accept_len + 1 on the device (one decode step's committed tokens).
struct AdvanceArgs {
  int64_t* pos;
  const int32_t* accept_len;
};
hipError_t launch_advance(const AdvanceArgs& a, hipStream_t stream);

struct ScatterArgs {
  const uint16_t* k_src;  // [n][Hkv][D]
  const uint16_t* v_src;
  int64_t pos_first, n;
  int32_t n_kv_heads, head_dim;
  uint16_t* k_dst;        // chunked store
  uint16_t* v_dst;
  const int32_t* pt;      // nullptr: ring
  int32_t n_table;        // page table entries (paged)
  int32_t n_slots;        // pool slots, or ring chunk slots
  int64_t ring_size;
  // append of a verify block to the pool: chunks first_new .. first_new+n_new-1 take
  // new_slots[] (and pt_w, the writable table, gets those entries); others read pt
  int32_t* pt_w;          // nullptr: no table writes
  int32_t first_new, n_new;
  int32_t new_slots[RKV_MAX_APPEND_CHUNKS];
  // device-resident first position (nullptr: pos_first holds); a value outside [0, pos_cap]
  // writes nothing
  const int64_t* d_pos;
  int64_t pos_cap;
};
hipError_t launch_scatter(const ScatterArgs& a, hipStream_t stream);

// Whole chunks between pool slots and the packed staging area of a host page-out / page-in.
struct PageArgs {
  uint8_t* pool_k;        // [n_slots][chunk_bytes]
  uint8_t* pool_v;
  uint8_t* stage;         // [2][n][chunk_bytes]: the K blocks, then the V blocks
  int64_t chunk_bytes;    // n_kv_heads * 64 * head_dim * 2, a multiple of 16
  int32_t n;              // chunks in this batch, 1 .. RKV_PAGE_BATCH
  int32_t to_stage;       // 1: pool -> staging, 0: staging -> pool
  int32_t slots[RKV_PAGE_BATCH];
};
hipError_t launch_page_copy(const PageArgs& a, hipStream_t stream);

// Whole chunks straight between pool slots and host entries, through the device-visible address
// of pinned host memory (for batches whose chunk ids are scattered).
struct PageHostArgs {
  uint8_t* pool_k;
  uint8_t* pool_v;
  uint8_t* host_k;        // device-visible address of the host store's entry 0
  uint8_t* host_v;
  int64_t chunk_bytes;
  int32_t n;
  int32_t to_host;        // 1: pool -> host, 0: host -> pool
  int32_t slots[RKV_PAGE_BATCH];
  int32_t chunk_ids[RKV_PAGE_BATCH];
};
hipError_t launch_page_host(const PageHostArgs& a, hipStream_t stream);

}  // namespace rkv
