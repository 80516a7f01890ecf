// Log-sum-exp merge of split-K attention partials.  A split's partial is its normalised
// output O_s and lse_s over its own keys; with M = max_s lse_s and w_s = exp(lse_s - M) the
// whole is sum_s w_s O_s / sum_s w_s and lse = M + ln sum_s w_s (a regrouping of the plain
// softmax over all keys; splits with lse_s = -inf saw no key of a row and carry no weight).
#include "rkv_device.hpp"
#include "rkv_launch.hpp"

namespace rkv {
namespace {

// One workgroup per (KV head, row), one thread per output dimension.  The splits are read in
// tiles of kTile with every load of a tile in flight at once (a split-by-split loop would wait
// one memory latency per split), and merged online: the running max only ever grows, and the
// running sums are rescaled when it does.
constexpr int kTile = 16;

__global__ __launch_bounds__(128) void merge_kernel(MergeArgs a) {
  const int rows = a.q_len * a.G;
  const int g = blockIdx.x / rows;
  const int r = blockIdx.x % rows;
  const int d = threadIdx.x;
  const int S = a.num_splits;
  const float* lse = a.part_lse + (int64_t)g * S * rows + r;
  const float* po = a.part_o + ((int64_t)g * S * rows + r) * a.head_dim + d;
  const int64_t ostride = (int64_t)rows * a.head_dim;

  float M = -INFINITY, sum = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < S; s0 += kTile) {
    float ls[kTile], ov[kTile];
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      // clamped index: every load is issued unconditionally, the tail is masked afterwards
      const int sj = min(s0 + j, S - 1);
      const float l = lse[(int64_t)sj * rows];
      const float o = po[sj * ostride];
      ls[j] = s0 + j < S ? l : -INFINITY;
      ov[j] = o;
    }
    float mt = M;
#pragma unroll
    for (int j = 0; j < kTile; ++j) mt = fmaxf(mt, ls[j]);
    if (mt == -INFINITY) continue;           // no split so far saw a key of this row
    const float rescale = expf(M - mt);      // M = -inf: 0, and sum = acc = 0 anyway
    sum *= rescale;
    acc *= rescale;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const float w = ls[j] > -INFINITY ? expf(ls[j] - mt) : 0.f;
      sum += w;
      acc = fmaf(w, ov[j], acc);
    }
    M = mt;
  }
  const int qi = r / a.G;
  const int h = g * a.G + r % a.G;
  a.out[((int64_t)qi * a.n_q_heads + h) * a.head_dim + d] = sum > 0.f ? acc / sum : 0.f;
  if (a.lse != nullptr && d == 0)
    a.lse[(int64_t)qi * a.n_q_heads + h] = sum > 0.f ? M + logf(sum) : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int blocks = a.n_kv_heads * a.q_len * a.G;
  hipLaunchKernelGGL(merge_kernel, dim3(blocks), dim3(a.head_dim), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rkv
