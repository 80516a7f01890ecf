// Contiguous rows -> chunked KV store (ring or paged pool); also the append of a verify block's
// own rows.  Position p of the rows goes to
// ring slot p mod ring_size (lucebox post "Laguna XS 2.1 33B on a RTX 3090: 296 tok/s peak,
// 152 tok/s at 256K context", "3. Ring caches for the sliding-window layers") or to pool slot
// page_table[p / 64] ("Three optimizations", item 1), offset p mod 64; K key-major and V
// dimension-major inside the chunk.  One thread per element.
#include "rkv_device.hpp"
#include "rkv_launch.hpp"

namespace rkv {
namespace {

__global__ __launch_bounds__(256) void scatter_kernel(ScatterArgs a) {
  const int64_t total = a.n * a.n_kv_heads * a.head_dim;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (a.pt_w != nullptr && e < a.n_new) a.pt_w[a.first_new + e] = a.new_slots[e];
  if (e >= total) return;
  const int d = (int)(e % a.head_dim);
  const int g = (int)((e / a.head_dim) % a.n_kv_heads);
  const int64_t i = e / ((int64_t)a.head_dim * a.n_kv_heads);
  int64_t pos_first = a.pos_first;
  if (a.d_pos != nullptr) {
    pos_first = *a.d_pos;
    if (pos_first < 0 || pos_first > a.pos_cap) return;
  }
  const int64_t pos = pos_first + i;
  int64_t slot, off;
  if (a.pt == nullptr) {
    const int64_t sl = pos % a.ring_size;
    slot = sl / kChunk;
    off = sl % kChunk;
  } else {
    const int64_t c = pos / kChunk;
    if (c >= a.n_table) return;
    // a chunk the appended block starts takes its new slot (its table entry is being
    // written by this launch); older chunks read the table
    slot = (a.pt_w != nullptr && c >= a.first_new) ? a.new_slots[c - a.first_new] : a.pt[c];
    if (slot < 0 || slot >= a.n_slots) return;
    off = pos % kChunk;
  }
  const int64_t blk = slot * a.n_kv_heads + g;
  a.k_dst[(blk * kChunk + off) * a.head_dim + d] = a.k_src[e];
  a.v_dst[(blk * a.head_dim + d) * kChunk + off] = a.v_src[e];
}

}  // namespace

hipError_t launch_scatter(const ScatterArgs& a, hipStream_t stream) {
  const int64_t total = a.n * a.n_kv_heads * a.head_dim;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  return launch_kernel(scatter_kernel, dim3((unsigned)blocks), dim3(256), a, stream);
}

}  // namespace rkv
