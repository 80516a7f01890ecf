// Greedy acceptance (lucebox post "Laguna XS 2.1 33B on a RTX 3090: 296 tok/s peak, 152 tok/s
// at 256K context", "TL;DR" and "The model, fast MoE with a drafter in the box": proposals are
// verified in one batched forward and what is committed is what greedy decoding by the
// target would produce).  Pass 1: every workgroup finds the first maximum of one (row, vocabulary part),
// reduced within a wave by shuffles and across waves through LDS.  Pass 2 (one workgroup):
// the parts reduce to the row argmaxes, then the first disagreement with the draft and the
// committed tokens.  Ties go to the lower index, values compare as float32 (-0 == +0).
// (A single launch that lets the last workgroup finish needs a device-scope release from
// every workgroup, which costs more here than the second launch; with the parts written and
// read by device-coherent stores and loads instead of a release, and an arrival counter, the
// accept over [17 x 65,536] took 10.7 us against 8.7 us for the two launches.)
#include <limits.h>

#include "rkv_device.hpp"
#include "rkv_launch.hpp"

namespace rkv {
namespace {

// (value, index) order: larger value first, then lower index; NaN never wins a comparison.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off, kWave);
    const int oi = __shfl_xor(bi, off, kWave);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
}

constexpr int kScan = 16;   // elements per thread per part: part_len <= 256 * kScan = 4096

template <bool VEC4>
__global__ __launch_bounds__(256) void accept_partial_kernel(AcceptArgs a) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int row = blockIdx.y, part = blockIdx.x, tid = threadIdx.x;
  const int start = part * a.part_len;
  const int end = min(start + a.part_len, a.vocab);
  const float* L = a.logits + (int64_t)row * a.vocab;
  float bv = -INFINITY;
  int bi = INT_MAX;
  // a part is at most kScan * 256 elements: every load of the scan is issued before the first
  // compare (clamped to the part; duplicates of the last element cannot win, they only tie
  // with a lower index of the same value)
  if (VEC4) {
    const f32x4* L4 = reinterpret_cast<const f32x4*>(L);
    f32x4 x[kScan / 4];
#pragma unroll
    for (int u = 0; u < kScan / 4; ++u) {
      const int v = min(start + 4 * tid + 1024 * u, end - 4);
      x[u] = L4[v >> 2];
    }
#pragma unroll
    for (int u = 0; u < kScan / 4; ++u) {
      const int v = min(start + 4 * tid + 1024 * u, end - 4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (better(x[u][e], v + e, bv, bi)) { bv = x[u][e]; bi = v + e; }
    }
  } else {
    float x[kScan];
#pragma unroll
    for (int u = 0; u < kScan; ++u) x[u] = L[min(start + tid + 256 * u, end - 1)];
#pragma unroll
    for (int u = 0; u < kScan; ++u) {
      const int v = min(start + tid + 256 * u, end - 1);
      if (better(x[u], v, bv, bi)) { bv = x[u]; bi = v; }
    }
  }
  wave_argmax(bv, bi);
  const int w = tid >> 6;
  if ((tid & 63) == 0) { sv[w] = bv; si[w] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < 4; ++k)
      if (better(sv[k], si[k], bv, bi)) { bv = sv[k]; bi = si[k]; }
    a.part_val[(int64_t)row * a.parts + part] = bv;
    a.part_idx[(int64_t)row * a.parts + part] = bi;
  }
}

// Pass 2 reduces each row's parts with a group of GP lanes (the part count rounded up to a power
// of two, at most 64), 256 / GP rows side by side; every thread issues its loads for kRounds such
// rounds before its first compare, so the step's 17 rows of 16 parts cost one memory round trip.
constexpr int kRounds = 4;

__global__ __launch_bounds__(256) void accept_final_kernel(AcceptArgs a) {
  __shared__ int t[256];
  __shared__ int prop[256];
  __shared__ int acc_len;
  const int tid = threadIdx.x;
  const int n_draft = a.n_rows - 1;
  // the draft token is loaded with the parts and written to LDS after them, so that its load
  // does not hold the part loads back by a round trip
  const int my_prop = n_draft > 0 ? a.proposals[min(tid, n_draft - 1)] : 0;   // clamped: in range
  int GP = 1;
  while (GP < a.parts && GP < 64) GP <<= 1;
  const int rpr = 256 / GP;                 // rows per round
  const int lg = tid % GP;                  // this lane's place in its row's group
  const bool more_parts = a.parts > GP;     // vocabularies above 64 x 4,096 only
  for (int r0 = 0; r0 < a.n_rows; r0 += rpr * kRounds) {
    float lv[kRounds];
    int li[kRounds];
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {     // clamped, so every load is in range and issued
      const int row = min(r0 + k * rpr + tid / GP, a.n_rows - 1);
      const int64_t off = (int64_t)row * a.parts + min(lg, a.parts - 1);
      lv[k] = a.part_val[off];
      li[k] = a.part_idx[off];
    }
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
      const int row = r0 + k * rpr + tid / GP;
      // selects rather than a branch, so that the loads above stay ahead of every compare
      const bool own = row < a.n_rows && lg < a.parts;
      float bv = own ? lv[k] : -INFINITY;
      int bi = own ? li[k] : INT_MAX;
      if (more_parts && row < a.n_rows) {
        for (int p = lg + GP; p < a.parts; p += GP) {
          const float v = a.part_val[(int64_t)row * a.parts + p];
          const int i = a.part_idx[(int64_t)row * a.parts + p];
          if (better(v, i, bv, bi)) { bv = v; bi = i; }
        }
      }
      for (int off = GP >> 1; off >= 1; off >>= 1) {   // within the aligned group of GP lanes
        const float ov = __shfl_xor(bv, off, kWave);
        const int oi = __shfl_xor(bi, off, kWave);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if (lg == 0 && row < a.n_rows) {
        const int ri = bi == INT_MAX ? 0 : bi;   // a row of NaNs only: any in-range index
        t[row] = ri;
        if (a.row_argmax != nullptr) a.row_argmax[row] = ri;
      }
    }
  }
  if (tid < n_draft) prop[tid] = my_prop;
  __syncthreads();
  if (tid == 0) {
    int acc = n_draft;
    for (int r = 0; r < n_draft; ++r)
      if (t[r] != prop[r]) { acc = r; break; }
    acc_len = acc;
    a.accept_len[0] = acc;
  }
  __syncthreads();
  const int acc = acc_len;
  if (tid < a.n_rows) a.committed[tid] = tid < acc ? prop[tid] : (tid == acc ? t[acc] : -1);
}

// The commit of one decode step on the device: the next block starts a + 1 positions later
// (the a accepted drafts and the target's own next token).
__global__ __launch_bounds__(64) void advance_kernel(AdvanceArgs a) {
  if (threadIdx.x == 0) a.pos[0] += (int64_t)a.accept_len[0] + 1;
}

}  // namespace

hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream) {
  const dim3 grid(a.parts, a.n_rows);
  const hipError_t e = (a.vocab & 3) == 0 && (a.part_len & 3) == 0
                           ? launch_kernel(accept_partial_kernel<true>, grid, dim3(256), a, stream)
                           : launch_kernel(accept_partial_kernel<false>, grid, dim3(256), a, stream);
  if (e != hipSuccess) return e;
  return launch_kernel(accept_final_kernel, dim3(1), dim3(256), a, stream);
}

hipError_t launch_advance(const AdvanceArgs& a, hipStream_t stream) {
  return launch_kernel(advance_kernel, dim3(1), dim3(64), a, stream);
}

}  // namespace rkv
