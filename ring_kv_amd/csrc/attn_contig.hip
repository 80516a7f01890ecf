// Verify-block attention over the contiguous reference layout K, V [ctx][Hkv][D], f32 or
// bf16 inputs, every arithmetic step in f32 on the vector ALUs.  It is the GPU-side
// reference the chunked stores are checked against (and plain decode with one query); the
// HBM-bound verify path is the MFMA kernel over the chunked stores.
//
// Workgroup = (KV head, split of whole 64-key tiles, tile of 64 rows); four threads per row.
#include "rkv_device.hpp"
#include "rkv_launch.hpp"

namespace rkv {
namespace {

template <typename TIn>
__device__ __forceinline__ float load_in(const TIn* p, int64_t i);
template <>
__device__ __forceinline__ float load_in<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_in<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <int D, typename TIn>
__global__ __launch_bounds__(256) void contig_attn_kernel(ContigArgs a) {
  __shared__ float Qs[64][D + 1];
  __shared__ float Ks[64][D + 1];
  __shared__ float Vs[64][D + 1];
  __shared__ float Ps[64][65];

  const TIn* q = static_cast<const TIn*>(a.q);
  const TIn* k = static_cast<const TIn*>(a.k);
  const TIn* v = static_cast<const TIn*>(a.v);
  const int tid = threadIdx.x;
  const int rl = tid >> 2;          // row within the tile
  const int sub = tid & 3;          // quarter of the keys (scores) / of the dims (output)
  const int g = blockIdx.x % a.n_kv_heads;
  const int s = blockIdx.x / a.n_kv_heads;
  const int G = a.G;
  const int rows = a.q_len * G;
  const int r = blockIdx.y * 64 + rl;
  const bool row_ok = r < rows;
  const int qi = row_ok ? r / G : 0;
  const int hq = g * G + (row_ok ? r % G : 0);
  const int64_t p_i = a.ctx_len - a.q_len + qi;
  const int64_t lo_i = a.window > 0 ? imax64(0, p_i - a.window + 1) : 0;

  for (int e = tid; e < 64 * D; e += 256) {
    const int rr = e / D, d = e % D;
    const int r2 = blockIdx.y * 64 + rr;
    float x = 0.f;
    if (r2 < rows) x = load_in<TIn>(q, ((int64_t)(r2 / G) * a.n_q_heads + g * G + r2 % G) * D + d);
    Qs[rr][d] = x;
  }

  const int64_t c_lo = a.c_first + (int64_t)s * a.cps;
  const int64_t c_hi = imin64(c_lo + a.cps, a.c_first + a.n_chunks);
  float m_run = -INFINITY, l_run = 0.f;
  float o[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) o[i] = 0.f;

  for (int64_t c = c_lo; c < c_hi; ++c) {
    const int64_t kbase = c * 64;
    __syncthreads();
    for (int e = tid; e < 64 * D; e += 256) {
      const int key = e / D, d = e % D;
      const int64_t j = kbase + key;
      float kx = 0.f, vx = 0.f;
      if (j < a.ctx_len) {
        const int64_t idx = (j * a.n_kv_heads + g) * D + d;
        kx = load_in<TIn>(k, idx);
        vx = load_in<TIn>(v, idx);
      }
      Ks[key][d] = kx;
      Vs[key][d] = vx;
    }
    __syncthreads();
    float sc[16];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int key = sub * 16 + kk;
      float dot = 0.f;
#pragma unroll 16
      for (int d = 0; d < D; ++d) dot = fmaf(Qs[rl][d], Ks[key][d], dot);
      const int64_t j = kbase + key;
      const bool vis = row_ok && j < a.ctx_len && j <= p_i && j >= lo_i;
      sc[kk] = vis ? dot * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sc[kk]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 2, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const float p = exp2f(sc[kk] - m_use);
      Ps[rl][sub * 16 + kk] = p;
      lsum += p;
    }
    l_run = l_run * alpha + lsum;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      float acc = o[i] * alpha;
      const int d = sub * (D / 4) + i;
#pragma unroll 16
      for (int key = 0; key < 64; ++key) acc = fmaf(Ps[rl][key], Vs[key][d], acc);
      o[i] = acc;
    }
  }

  float l = l_run;
  l += __shfl_xor(l, 1, kWave);
  l += __shfl_xor(l, 2, kWave);
  if (!row_ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse_nat = l > 0.f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
  float* dst;
  if (a.part_o == nullptr) {
    dst = a.out + ((int64_t)qi * a.n_q_heads + hq) * D;
    if (a.lse != nullptr && sub == 0) a.lse[(int64_t)qi * a.n_q_heads + hq] = lse_nat;
  } else {
    const int64_t prow = ((int64_t)g * a.num_splits + s) * rows + r;
    dst = a.part_o + prow * D;
    if (sub == 0) a.part_lse[prow] = lse_nat;
  }
#pragma unroll
  for (int i = 0; i < D / 4; ++i) dst[sub * (D / 4) + i] = o[i] * inv;
}

template <int D>
hipError_t launch_d(const ContigArgs& a, hipStream_t stream) {
  const int rows = a.q_len * a.G;
  const dim3 grid(a.n_kv_heads * a.num_splits, (rows + 63) / 64);
  if (a.dtype == 1)
    hipLaunchKernelGGL((contig_attn_kernel<D, uint16_t>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((contig_attn_kernel<D, float>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_contig_attn(const ContigArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  return launch_d<64>(a, stream);
}

}  // namespace rkv
