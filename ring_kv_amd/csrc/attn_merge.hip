// Log-sum-exp merge of split-K attention partials.  A split's partial is its normalised
// output O_s and lse_s over its own keys; with M = max_s lse_s and w_s = exp(lse_s - M) the
// whole is sum_s w_s O_s / sum_s w_s and lse = M + ln sum_s w_s (a regrouping of the plain
// softmax over all keys; splits with lse_s = -inf saw no key of a row and carry no weight).
// A NaN partial (a split that refused its input) makes the row NaN: it is never dropped.
// The pages split no key range; the split over chunk ranges is this library's way of spreading
// one long-context verify block over all compute units.
#include "rkv_device.hpp"
#include "rkv_launch.hpp"

namespace rkv {
namespace {

// Few rows, many splits (a verify block over a long context): one workgroup of 256 threads per
// (KV head, row).  Thread (sg, d4) owns four consecutive output dimensions and the splits sg,
// sg + SG, ...; its first kPre partial vectors are requested before anything else so that the
// whole merge costs about one memory round trip.
// The max over the splits' lse values is reduced through LDS, then every thread weighs its
// splits, and the SG split groups are summed through LDS.
constexpr int kMergeThreads = 256;
constexpr int kPre = 8;

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  v = red[0];
  for (int k = 1; k < kMergeThreads / 64; ++k) v = fmaxf(v, red[k]);
  return v;
}

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  constexpr int PR = D / 4;                 // float4 per row
  constexpr int SG = kMergeThreads / PR;    // split groups
  static_assert(SG == merge_groups<D>(), "the split grouping every merge path shares");
  __shared__ float red[kMergeThreads / 64];
  __shared__ f32x4 xacc[SG][PR];
  __shared__ float xl[SG];

  const int rows = a.q_len * a.G;
  const int g = blockIdx.x / rows;
  const int r = blockIdx.x % rows;
  const int tid = threadIdx.x;
  const int sg = tid / PR;
  const int d4 = (tid % PR) * 4;
  const int S = a.num_splits;
  const float* lse = a.part_lse + (int64_t)g * S * rows + r;
  const float* po = a.part_o + ((int64_t)g * S * rows + r) * D + d4;
  const int64_t ostride = (int64_t)rows * D;

  f32x4 ov[kPre];
  float lv[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int sj = min(sg + SG * u, S - 1);     // clamped: every load is in range and issued
    ov[u] = *reinterpret_cast<const f32x4*>(po + sj * ostride);
    lv[u] = lse[(int64_t)sj * rows];
  }
  float mloc = -INFINITY;
  for (int s = tid; s < S; s += kMergeThreads) mloc = fmaxf(mloc, lse[(int64_t)s * rows]);
  const float M = block_max(mloc, red);
  const float Mu = M == -INFINITY ? 0.f : M;      // no split saw a key: everything weighs 0

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
#pragma unroll
  for (int u = 0; u < kPre; ++u)
    if (sg + SG * u < S) merge_term(acc, L, ov[u], lv[u], Mu);
  for (int s = sg + SG * kPre; s < S; s += SG)
    merge_term(acc, L, *reinterpret_cast<const f32x4*>(po + s * ostride),
               lse[(int64_t)s * rows], Mu);
  xacc[sg][tid % PR] = acc;
  if (tid % PR == 0) xl[sg] = L;
  __syncthreads();
  if (sg != 0) return;
  float Lt = 0.f;
  for (int k = 0; k < SG; ++k) {
    Lt += xl[k];
    if (k) acc += xacc[k][tid % PR];
  }
  const int qi = r / a.G;
  const int h = g * a.G + r % a.G;
  *reinterpret_cast<f32x4*>(a.out + ((int64_t)qi * a.n_q_heads + h) * D + d4) =
      merge_out(acc, Lt);
  if (a.lse != nullptr && d4 == 0) a.lse[(int64_t)qi * a.n_q_heads + h] = merge_lse(M, Lt);
}

// Many rows, few splits (a prefill block): D/4 threads per row, each owning four consecutive
// dimensions and walking the splits group by group (merge_kernel's grouping, so the same bits);
// no LDS, no barrier, and each row's partials are read as whole 4*D-byte lines.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_rows_kernel(MergeArgs a) {
  constexpr int TPR = D / 4;
  constexpr int RPB = kMergeThreads / TPR;
  const int rows = a.q_len * a.G;
  const int64_t gr = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  if (gr >= (int64_t)a.n_kv_heads * rows) return;
  const int g = (int)(gr / rows);
  const int r = (int)(gr % rows);
  const int d4 = (threadIdx.x % TPR) * 4;
  const int S = a.num_splits;
  const float* lse = a.part_lse + (int64_t)g * S * rows + r;
  const float* po = a.part_o + ((int64_t)g * S * rows + r) * D + d4;
  const int64_t ostride = (int64_t)rows * D;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, lse[(int64_t)s * rows]);
  const float Mu = M == -INFINITY ? 0.f : M;
  // the split groups of merge_kernel, one after the other (the same bits)
  constexpr int SG = merge_groups<D>();
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float Lt = 0.f;
  for (int sg = 0; sg < SG; ++sg) {
    f32x4 acc_g = f32x4{0.f, 0.f, 0.f, 0.f};
    float L_g = 0.f;
    for (int s = sg; s < S; s += SG)
      merge_term(acc_g, L_g, *reinterpret_cast<const f32x4*>(po + s * ostride),
                 lse[(int64_t)s * rows], Mu);
    Lt += L_g;
    if (sg == 0) acc = acc_g;
    else acc += acc_g;
  }
  const int qi = r / a.G;
  const int h = g * a.G + r % a.G;
  *reinterpret_cast<f32x4*>(a.out + ((int64_t)qi * a.n_q_heads + h) * D + d4) =
      merge_out(acc, Lt);
  if (a.lse != nullptr && d4 == 0) a.lse[(int64_t)qi * a.n_q_heads + h] = merge_lse(M, Lt);
}

// rows of all KV heads from which the row-parallel form is used (with at most kRowsMaxSplits)
constexpr int64_t kRowsMinRows = 1024;
constexpr int kRowsMaxSplits = 32;

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int64_t all_rows = (int64_t)a.n_kv_heads * a.q_len * a.G;
  if (all_rows >= kRowsMinRows && a.num_splits <= kRowsMaxSplits) {
    const int rpb = kMergeThreads / (a.head_dim / 4);
    const dim3 blocks((unsigned)((all_rows + rpb - 1) / rpb));
    if (a.head_dim == 128)
      return launch_kernel(merge_rows_kernel<128>, blocks, dim3(kMergeThreads), a, stream);
    return launch_kernel(merge_rows_kernel<64>, blocks, dim3(kMergeThreads), a, stream);
  }
  const int blocks = (int)all_rows;
  if (a.head_dim == 128)
    return launch_kernel(merge_kernel<128>, dim3(blocks), dim3(kMergeThreads), a, stream);
  return launch_kernel(merge_kernel<64>, dim3(blocks), dim3(kMergeThreads), a, stream);
}

}  // namespace rkv
