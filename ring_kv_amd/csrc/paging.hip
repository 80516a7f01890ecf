// Host paging of the pool: whole 64-token chunks copied between pool slots and a host chunk
// store, bit-exact (lucebox post "Laguna XS 2.1 33B on a RTX 3090: 296 tok/s peak, 152 tok/s at
// 256K context", "Three optimizations", item 1: chunks move between the pool and host memory).
//
// A chunk's K and V are each one contiguous block of n_kv_heads * 64 * head_dim bf16 in a slot,
// so the copies need no layout change.  Two paths, chosen per batch:
//  * long runs of consecutive chunk ids, or a store the device cannot address: the chunks are
//    packed into a device staging area by a kernel (HBM to HBM) and cross PCIe with the copy
//    engines, one copy per run;
//  * a pinned host store, for every page-out and for page-ins of scattered chunk ids (where one
//    copy per run would pay the copy engines' per-copy cost many times): a kernel copies every
//    chunk straight between its slot and its host entry, through the address the runtime maps
//    for the device (hipHostGetDevicePointer; memory it cannot map always takes the first path).
#include <algorithm>
#include <vector>

#include "../../include/ring_kv.h"
#include "rkv_device.hpp"
#include "rkv_launch.hpp"

namespace rkv {
namespace {

constexpr int kPageThreads = 256;

// Entry e < n is the K block of slots[e], entry n + e its V block; staging entry e sits at
// stage + e * chunk_bytes.  to_stage: pool -> staging (page-out), else staging -> pool.
__global__ __launch_bounds__(kPageThreads) void page_copy_kernel(PageArgs a) {
  const int e = blockIdx.x;
  const int i = e % a.n;
  uint8_t* pool = (e < a.n ? a.pool_k : a.pool_v) + (int64_t)a.slots[i] * a.chunk_bytes;
  uint8_t* stage = a.stage + (int64_t)e * a.chunk_bytes;
  const u32x4* src = reinterpret_cast<const u32x4*>(a.to_stage ? pool : stage);
  u32x4* dst = reinterpret_cast<u32x4*>(a.to_stage ? stage : pool);
  const int64_t n16 = a.chunk_bytes / 16;
  for (int64_t u = (int64_t)blockIdx.y * kPageThreads + threadIdx.x; u < n16;
       u += (int64_t)gridDim.y * kPageThreads)
    dst[u] = src[u];
}

// Entry e < n is the K block of chunk e, entry n + e its V block, copied between pool slot
// slots[e] and host entry chunk_ids[e].  Each thread keeps kUnroll 16-byte loads in flight before
// its stores: reads across PCIe take microseconds, and only many requests in flight fill the link.
constexpr int kUnroll = 4;
__global__ __launch_bounds__(kPageThreads) void page_host_kernel(PageHostArgs a) {
  const int e = blockIdx.x;
  const int i = e % a.n;
  const bool v = e >= a.n;
  uint8_t* pool = (v ? a.pool_v : a.pool_k) + (int64_t)a.slots[i] * a.chunk_bytes;
  uint8_t* host = (v ? a.host_v : a.host_k) + (int64_t)a.chunk_ids[i] * a.chunk_bytes;
  const u32x4* src = reinterpret_cast<const u32x4*>(a.to_host ? pool : host);
  u32x4* dst = reinterpret_cast<u32x4*>(a.to_host ? host : pool);
  const int64_t n16 = a.chunk_bytes / 16;
  const int64_t step = (int64_t)gridDim.y * kPageThreads;
  for (int64_t u0 = (int64_t)blockIdx.y * kPageThreads + threadIdx.x; u0 < n16;
       u0 += step * kUnroll) {
    u32x4 r[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k)
      if (u0 + k * step < n16) r[k] = src[u0 + k * step];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k)
      if (u0 + k * step < n16) dst[u0 + k * step] = r[k];
  }
}

}  // namespace

hipError_t launch_page_host(const PageHostArgs& a, hipStream_t stream) {
  const int64_t n16 = a.chunk_bytes / 16;
  const int parts = (int)std::min<int64_t>(8, (n16 + kPageThreads - 1) / kPageThreads);
  return launch_kernel(page_host_kernel, dim3(2 * a.n, parts), dim3(kPageThreads), a, stream);
}

hipError_t launch_page_copy(const PageArgs& a, hipStream_t stream) {
  const int64_t n16 = a.chunk_bytes / 16;
  const int parts = (int)std::min<int64_t>(8, (n16 + kPageThreads - 1) / kPageThreads);
  return launch_kernel(page_copy_kernel, dim3(2 * a.n, parts), dim3(kPageThreads), a, stream);
}

}  // namespace rkv

namespace {

int64_t chunk_bytes_of(int32_t n_kv_heads, int32_t head_dim) {
  return (int64_t)n_kv_heads * RKV_CHUNK * head_dim * 2;
}

bool bad_shape(int32_t n_kv_heads, int32_t head_dim) {
  return n_kv_heads < 1 || (head_dim != 64 && head_dim != 128);
}

bool has_repeats(const int32_t* v, int32_t n) {
  std::vector<int32_t> s(v, v + n);
  std::sort(s.begin(), s.end());
  return std::adjacent_find(s.begin(), s.end()) != s.end();
}

// Checks shared by both directions (before any HIP call).
int32_t check_paging(int32_t n_kv_heads, int32_t head_dim, int32_t n_slots, const int32_t* slots,
                     const int32_t* chunk_ids, int32_t n, int64_t n_host, bool out,
                     const void* workspace, size_t workspace_bytes) {
  if (bad_shape(n_kv_heads, head_dim)) return RKV_ERR_SHAPE;
  if (n < 0 || n_host < 0) return RKV_ERR_ARG;
  if (n == 0) return RKV_OK;
  if (slots == nullptr || chunk_ids == nullptr) return RKV_ERR_NULL;
  for (int32_t i = 0; i < n; ++i) {
    if (chunk_ids[i] < 0 || chunk_ids[i] >= n_host) return RKV_ERR_ARG;
    if (slots[i] < 0 || slots[i] >= n_slots) return RKV_ERR_TABLE;
  }
  if (has_repeats(out ? chunk_ids : slots, n)) return RKV_ERR_ARG;
  if (workspace == nullptr || workspace_bytes < kv_page_workspace_bytes(n_kv_heads, head_dim, n))
    return RKV_ERR_WORKSPACE;
  return RKV_OK;
}

// One copy per run of consecutive chunk ids within batch [b0, b1): host entry chunk_ids[i] <->
// staging entry (i - b0) for K, and (nb + i - b0) for V.
hipError_t copy_runs(const int32_t* chunk_ids, int32_t b0, int32_t b1, uint8_t* stage,
                     uint8_t* k_host, uint8_t* v_host, int64_t cb, bool to_host, hipStream_t st) {
  const int32_t nb = b1 - b0;
  for (int32_t i = b0; i < b1;) {
    int32_t j = i + 1;
    while (j < b1 && chunk_ids[j] == chunk_ids[j - 1] + 1) ++j;
    const size_t bytes = (size_t)(j - i) * (size_t)cb;
    uint8_t* hk = k_host + (int64_t)chunk_ids[i] * cb;
    uint8_t* hv = v_host + (int64_t)chunk_ids[i] * cb;
    uint8_t* sk = stage + (int64_t)(i - b0) * cb;
    uint8_t* sv = stage + (int64_t)(nb + i - b0) * cb;
    hipError_t e;
    if (to_host) {
      e = hipMemcpyAsync(hk, sk, bytes, hipMemcpyDeviceToHost, st);
      if (e == hipSuccess) e = hipMemcpyAsync(hv, sv, bytes, hipMemcpyDeviceToHost, st);
    } else {
      e = hipMemcpyAsync(sk, hk, bytes, hipMemcpyHostToDevice, st);
      if (e == hipSuccess) e = hipMemcpyAsync(sv, hv, bytes, hipMemcpyHostToDevice, st);
    }
    if (e != hipSuccess) return e;
    i = j;
  }
  return hipSuccess;
}

// Runs of consecutive chunk ids in batch [b0, b1).
int32_t count_runs(const int32_t* chunk_ids, int32_t b0, int32_t b1) {
  int32_t runs = 1;
  for (int32_t i = b0 + 1; i < b1; ++i) runs += chunk_ids[i] != chunk_ids[i - 1] + 1;
  return runs;
}

// With a host store the device can address (pinned memory), a page-out always takes the direct
// kernel (measured: 310 µs for 128 chunks in one run against 327 µs through staging and the copy
// engines, the same for scattered ids), and a page-in takes it for scattered ids (runs shorter
// than kMinRun chunks on average: 353 µs for 128 scattered chunks against ~2.5 ms for one copy
// per run); a page-in of long runs goes through the copy engines (329 µs against 357 µs).
constexpr int32_t kMinRun = 8;

// Device-visible addresses of the two host stores, or false when either is not pinned memory
// mapped for the device (then only the copy engines touch it).
bool host_device_ptrs(const void* k_host, const void* v_host, uint8_t** dk, uint8_t** dv) {
  void* a = nullptr;
  void* b = nullptr;
  if (hipHostGetDevicePointer(&a, const_cast<void*>(k_host), 0) != hipSuccess ||
      hipHostGetDevicePointer(&b, const_cast<void*>(v_host), 0) != hipSuccess) {
    (void)hipGetLastError();   // the query failed; leave no error for the next call to report
    return false;
  }
  *dk = static_cast<uint8_t*>(a);
  *dv = static_cast<uint8_t*>(b);
  return true;
}

hipError_t direct_batch(void* k_pool, void* v_pool, uint8_t* dk, uint8_t* dv, int64_t cb,
                        const int32_t* slots, const int32_t* chunk_ids, int32_t b0, int32_t b1,
                        bool to_host, hipStream_t st) {
  rkv::PageHostArgs a{};
  a.pool_k = static_cast<uint8_t*>(k_pool);
  a.pool_v = static_cast<uint8_t*>(v_pool);
  a.host_k = dk;
  a.host_v = dv;
  a.chunk_bytes = cb;
  a.n = b1 - b0;
  a.to_host = to_host ? 1 : 0;
  for (int32_t i = b0; i < b1; ++i) {
    a.slots[i - b0] = slots[i];
    a.chunk_ids[i - b0] = chunk_ids[i];
  }
  return rkv::launch_page_host(a, st);
}

rkv::PageArgs batch_args(void* k_pool, void* v_pool, void* workspace, int64_t cb,
                         const int32_t* slots, int32_t b0, int32_t b1, bool to_stage) {
  rkv::PageArgs a{};
  a.pool_k = static_cast<uint8_t*>(k_pool);
  a.pool_v = static_cast<uint8_t*>(v_pool);
  a.stage = static_cast<uint8_t*>(workspace);
  a.chunk_bytes = cb;
  a.n = b1 - b0;
  a.to_stage = to_stage ? 1 : 0;
  for (int32_t i = b0; i < b1; ++i) a.slots[i - b0] = slots[i];
  return a;
}

}  // namespace

extern "C" {

size_t kv_page_workspace_bytes(int32_t n_kv_heads, int32_t head_dim, int32_t n) {
  if (bad_shape(n_kv_heads, head_dim) || n <= 0) return 0;
  const int64_t nb = std::min<int32_t>(n, RKV_PAGE_BATCH);
  return (size_t)(2 * nb * chunk_bytes_of(n_kv_heads, head_dim));
}

int32_t kv_page_out(const void* k_pool, const void* v_pool, int32_t n_kv_heads,
                    int32_t head_dim, int32_t n_slots, const int32_t* slots,
                    const int32_t* chunk_ids, int32_t n, void* k_host, void* v_host,
                    int64_t n_host, void* workspace, size_t workspace_bytes, void* stream) {
  if (k_pool == nullptr || v_pool == nullptr || k_host == nullptr || v_host == nullptr)
    return RKV_ERR_NULL;
  int32_t st = check_paging(n_kv_heads, head_dim, n_slots, slots, chunk_ids, n, n_host, true,
                            workspace, workspace_bytes);
  if (st != RKV_OK || n == 0) return st;
  const int64_t cb = chunk_bytes_of(n_kv_heads, head_dim);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  uint8_t *dk = nullptr, *dv = nullptr;
  const bool direct_ok = host_device_ptrs(k_host, v_host, &dk, &dv);
  for (int32_t b0 = 0; b0 < n; b0 += RKV_PAGE_BATCH) {
    const int32_t b1 = std::min<int32_t>(n, b0 + RKV_PAGE_BATCH);
    if (direct_ok) {
      if (direct_batch(const_cast<void*>(k_pool), const_cast<void*>(v_pool), dk, dv, cb, slots,
                       chunk_ids, b0, b1, true, hs) != hipSuccess)
        return RKV_ERR_HIP;
      continue;
    }
    rkv::PageArgs a = batch_args(const_cast<void*>(k_pool), const_cast<void*>(v_pool), workspace,
                                 cb, slots, b0, b1, true);
    hipError_t e = rkv::launch_page_copy(a, hs);
    if (e == hipSuccess)
      e = copy_runs(chunk_ids, b0, b1, static_cast<uint8_t*>(workspace),
                    static_cast<uint8_t*>(k_host), static_cast<uint8_t*>(v_host), cb, true, hs);
    if (e != hipSuccess) return RKV_ERR_HIP;
  }
  return RKV_OK;
}

int32_t kv_page_in(const void* k_host, const void* v_host, int64_t n_host,
                   const int32_t* chunk_ids, const int32_t* slots, int32_t n, void* k_pool,
                   void* v_pool, int32_t n_kv_heads, int32_t head_dim, int32_t n_slots,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (k_pool == nullptr || v_pool == nullptr || k_host == nullptr || v_host == nullptr)
    return RKV_ERR_NULL;
  int32_t st = check_paging(n_kv_heads, head_dim, n_slots, slots, chunk_ids, n, n_host, false,
                            workspace, workspace_bytes);
  if (st != RKV_OK || n == 0) return st;
  const int64_t cb = chunk_bytes_of(n_kv_heads, head_dim);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  uint8_t *dk = nullptr, *dv = nullptr;
  const bool direct_ok = host_device_ptrs(k_host, v_host, &dk, &dv);
  for (int32_t b0 = 0; b0 < n; b0 += RKV_PAGE_BATCH) {
    const int32_t b1 = std::min<int32_t>(n, b0 + RKV_PAGE_BATCH);
    if (direct_ok && count_runs(chunk_ids, b0, b1) * kMinRun > b1 - b0) {
      if (direct_batch(k_pool, v_pool, dk, dv, cb, slots, chunk_ids, b0, b1, false, hs) !=
          hipSuccess)
        return RKV_ERR_HIP;
      continue;
    }
    hipError_t e = copy_runs(chunk_ids, b0, b1, static_cast<uint8_t*>(workspace),
                             static_cast<uint8_t*>(const_cast<void*>(k_host)),
                             static_cast<uint8_t*>(const_cast<void*>(v_host)), cb, false, hs);
    if (e == hipSuccess) {
      rkv::PageArgs a = batch_args(k_pool, v_pool, workspace, cb, slots, b0, b1, false);
      e = rkv::launch_page_copy(a, hs);
    }
    if (e != hipSuccess) return RKV_ERR_HIP;
  }
  return RKV_OK;
}

}  // extern "C"
