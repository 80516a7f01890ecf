// Contiguous rows -> chunked KV store (ring or paged pool); also the append of a verify block's
// own rows.  Position p of the rows goes to
// ring slot p mod ring_size (lucebox post "Laguna XS 2.1 33B on a RTX 3090: 296 tok/s peak,
// 152 tok/s at 256K context", "3. Ring caches for the sliding-window layers") or to pool slot
// page_table[p / 64] ("Three optimizations", item 1), offset p mod 64; K key-major and V
// dimension-major inside the chunk.
//
// Blocks of more than 64 rows (a prefill block, a whole context): one workgroup per (chunk the
// rows touch, KV head).  K rows keep their layout (a position's D values stay contiguous), so they
// go straight from the source to the slot with 16-byte loads and stores.  V turns from
// position-major rows into dimension-major chunk rows: the workgroup reads its rows with 16-byte
// loads, transposes them through LDS, and writes each dimension's run of positions with 16-byte
// stores (eight positions each), so that both the reads and the writes are contiguous; positions
// of the chunk outside the rows are left as they are.  A verify block's 16 rows touch at most 16
// positions of a chunk row: there one thread per element and no LDS or barrier is quicker (2.2
// against 2.5 us per append in a graph; 1,024 rows: 5.4 against 3.2 us).
#include "rkv_device.hpp"
#include "rkv_launch.hpp"

namespace rkv {
namespace {

constexpr int kScatterThreads = 256;

// LDS place of (dimension d, chunk offset o) in the V transpose: rows of 64 positions whose
// 16-byte groups are XOR-swizzled by d / 8, so that the transposing 2-byte writes of the 16 lanes
// that share a position fall into different banks.
__device__ __forceinline__ int vt_at(int d, int o) {
  return d * kChunk + ((((o >> 3) ^ (d >> 3)) & 7) << 3) + (o & 7);
}

// The slot of logical chunk c, or -1 (no slot: its rows are skipped).
__device__ __forceinline__ int64_t slot_of_chunk(const ScatterArgs& a, int64_t c) {
  if (a.pt == nullptr) return c % a.n_slots;     // ring: position p at slot p mod ring_size
  if (c >= a.n_table) return -1;
  // a chunk the appended block starts takes its new slot (its table entry is being written by
  // this launch); older chunks read the table
  const int64_t slot = (a.pt_w != nullptr && c >= a.first_new) ? a.new_slots[c - a.first_new]
                                                                : a.pt[c];
  return (slot < 0 || slot >= a.n_slots) ? -1 : slot;
}

__device__ __forceinline__ bool device_pos(const ScatterArgs& a, int64_t* pos_first) {
  *pos_first = a.pos_first;
  if (a.d_pos == nullptr) return true;
  *pos_first = *a.d_pos;
  return *pos_first >= 0 && *pos_first <= a.pos_cap;
}

// few rows: one thread per element (i, g, d)
__global__ __launch_bounds__(kScatterThreads) void scatter_rows_kernel(ScatterArgs a) {
  const int64_t total = a.n * a.n_kv_heads * a.head_dim;
  const int64_t e = (int64_t)blockIdx.x * kScatterThreads + threadIdx.x;
  if (a.pt_w != nullptr && e < a.n_new) a.pt_w[a.first_new + e] = a.new_slots[e];
  int64_t pos_first;
  if (e >= total || !device_pos(a, &pos_first)) return;
  const int d = (int)(e % a.head_dim);
  const int g = (int)((e / a.head_dim) % a.n_kv_heads);
  const int64_t pos = pos_first + e / ((int64_t)a.head_dim * a.n_kv_heads);
  const int64_t slot = slot_of_chunk(a, pos / kChunk);
  if (slot < 0) return;
  const int64_t off = pos % kChunk;
  const int64_t blk = slot * a.n_kv_heads + g;
  a.k_dst[(blk * kChunk + off) * a.head_dim + d] = a.k_src[e];
  a.v_dst[(blk * a.head_dim + d) * kChunk + off] = a.v_src[e];
}

template <int D>
__global__ __launch_bounds__(kScatterThreads) void scatter_kernel(ScatterArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * kChunk];
  const int tid = threadIdx.x;
  if (a.pt_w != nullptr && blockIdx.x == 0 && tid < a.n_new)
    a.pt_w[a.first_new + tid] = a.new_slots[tid];
  int64_t pos_first;
  if (!device_pos(a, &pos_first)) return;
  const int g = blockIdx.x % a.n_kv_heads;
  const int64_t c = pos_first / kChunk + blockIdx.x / a.n_kv_heads;   // logical chunk
  const int64_t lo = imax64(pos_first, c * kChunk);
  const int64_t hi = imin64(pos_first + a.n, (c + 1) * kChunk);
  if (lo >= hi) return;                    // past the rows (grids sized for any alignment)
  const int64_t slot = slot_of_chunk(a, c);
  if (slot < 0) return;
  const int o0 = (int)(lo - c * kChunk);   // first and last+1 offsets in the chunk
  const int o1 = (int)(hi - c * kChunk);
  const int cnt = o1 - o0;
  constexpr int P8 = D / 8;                // 16-byte pieces per row
  const int64_t src_row = (int64_t)a.n_kv_heads * D;
  const int64_t i0 = lo - pos_first;       // source row of offset o0
  const int64_t blk = slot * a.n_kv_heads + g;
  uint16_t* kd = a.k_dst + blk * (kChunk * D);
  uint16_t* vd = a.v_dst + blk * (kChunk * D);
  for (int u = tid; u < cnt * P8; u += kScatterThreads) {
    const int j = u / P8, p = u % P8;
    const int64_t src = (i0 + j) * src_row + (int64_t)g * D + 8 * p;
    const u32x4 kv = *reinterpret_cast<const u32x4*>(a.k_src + src);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(a.v_src + src);
    *reinterpret_cast<u32x4*>(kd + (o0 + j) * D + 8 * p) = kv;
    // V: the eight dimensions 8p .. 8p+7 of position o0 + j into column o0 + j of the transpose
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vt[vt_at(8 * p + 2 * e, o0 + j)] = (uint16_t)(vv[e] & 0xffffu);
      vt[vt_at(8 * p + 2 * e + 1, o0 + j)] = (uint16_t)(vv[e] >> 16);
    }
  }
  __syncthreads();
  // V^T rows: dimension d, positions in groups of eight; whole groups go out as 16-byte stores,
  // a group the rows cover in part goes out element by element
  for (int u = tid; u < D * (kChunk / 8); u += kScatterThreads) {
    const int d = u / (kChunk / 8), q = u % (kChunk / 8);
    const int b0 = 8 * q, b1 = b0 + 8;
    if (b1 <= o0 || b0 >= o1) continue;
    if (b0 >= o0 && b1 <= o1) {
      *reinterpret_cast<u32x4*>(vd + d * kChunk + b0) =
          *reinterpret_cast<const u32x4*>(&vt[vt_at(d, b0)]);
    } else {
      for (int o = max(b0, o0); o < min(b1, o1); ++o) vd[d * kChunk + o] = vt[vt_at(d, o)];
    }
  }
}

}  // namespace

hipError_t launch_scatter(const ScatterArgs& a, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  if (a.n <= 64) {
    const int64_t total = a.n * a.n_kv_heads * a.head_dim;
    const dim3 grid((unsigned)((total + kScatterThreads - 1) / kScatterThreads));
    return launch_kernel(scatter_rows_kernel, grid, dim3(kScatterThreads), a, stream);
  }
  // chunks n rows can touch at any alignment of their first position
  const int64_t chunks = (a.n + kChunk - 2) / kChunk + 1;
  const dim3 grid((unsigned)(chunks * a.n_kv_heads));
  if (a.head_dim == 128) return launch_kernel(scatter_kernel<128>, grid, dim3(kScatterThreads), a, stream);
  return launch_kernel(scatter_kernel<64>, grid, dim3(kScatterThreads), a, stream);
}

}  // namespace rkv
