// Greedy acceptance (lucebox post "Laguna XS 2.1 33B on a RTX 3090: 296 tok/s peak, 152 tok/s
// at 256K context", "TL;DR" and "The model, fast MoE with a drafter in the box": proposals are
// verified in one batched forward and only tokens the target itself would emit are
// committed).  One launch: every workgroup finds the first maximum of one (row, vocabulary
// part), reduced within a wave by shuffles and across waves through LDS, publishes it, and
// takes a ticket; the workgroup that takes the last ticket reduces the parts to the row
// argmaxes, finds the first disagreement with the draft, writes the committed tokens and
// resets the ticket.  Ties go to the lower index, values compare as float32 (-0 == +0).
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

template <bool VEC4>
__global__ __launch_bounds__(256) void accept_kernel(AcceptArgs a) {
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ int last;
  __shared__ int t[256];
  __shared__ int acc_len;
  const int row = blockIdx.y, part = blockIdx.x, tid = threadIdx.x;
  const int start = part * a.part_len;
  const int end = min(start + a.part_len, a.vocab);
  const float* L = a.logits + (int64_t)row * a.vocab;
  float bv = -INFINITY;
  int bi = INT_MAX;
  if (VEC4) {
    // start and the row are 16-byte aligned (vocab and part_len are multiples of 4)
    const f32x4* L4 = reinterpret_cast<const f32x4*>(L);
    for (int v = start + 4 * tid; v < end; v += 4 * 256) {
      const f32x4 x = L4[v >> 2];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (better(x[e], v + e, bv, bi)) { bv = x[e]; bi = v + e; }
    }
  } else {
    for (int v = start + tid; v < end; v += 256) {
      const float x = L[v];
      if (better(x, v, bv, bi)) { bv = x; bi = v; }
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
    // release: this part is visible device-wide before the ticket is taken
    __threadfence();
    const unsigned total = (unsigned)(a.parts * a.n_rows);
    last = atomicAdd(a.ticket, 1u) == total - 1;
  }
  __syncthreads();
  if (!last) return;
  // acquire: every other workgroup's part is visible to this one
  __threadfence();
  const int n_draft = a.n_rows - 1;
  if (tid < a.n_rows) {
    float rv = -INFINITY;
    int ri = INT_MAX;
    for (int p = 0; p < a.parts; ++p) {
      const float v = __builtin_nontemporal_load(&a.part_val[(int64_t)tid * a.parts + p]);
      const int i = __builtin_nontemporal_load(&a.part_idx[(int64_t)tid * a.parts + p]);
      if (better(v, i, rv, ri)) { rv = v; ri = i; }
    }
    if (ri == INT_MAX) ri = 0;   // a row of NaNs only: any in-range index
    t[tid] = ri;
    if (a.row_argmax != nullptr) a.row_argmax[tid] = ri;
  }
  __syncthreads();
  if (tid == 0) {
    int acc = n_draft;
    for (int r = 0; r < n_draft; ++r)
      if (t[r] != a.proposals[r]) { acc = r; break; }
    acc_len = acc;
    a.accept_len[0] = acc;
    *a.ticket = 0u;             // ready for the next call
  }
  __syncthreads();
  const int acc = acc_len;
  if (tid < a.n_rows) a.committed[tid] = tid < acc ? a.proposals[tid] : (tid == acc ? t[acc] : -1);
}

}  // namespace

hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream) {
  const dim3 grid(a.parts, a.n_rows);
  if ((a.vocab & 3) == 0 && (a.part_len & 3) == 0)
    hipLaunchKernelGGL(accept_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(accept_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rkv
