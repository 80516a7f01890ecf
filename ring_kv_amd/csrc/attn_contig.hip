// Verify-block attention over the contiguous reference layout K, V [ctx][Hkv][D], f32 or
// bf16 inputs, every arithmetic step in f32: the products on the f32 matrix cores
// (v_mfma_f32_16x16x4_f32), the softmax on the vector ALUs.  It is the GPU-side reference the
// chunked stores are checked against (and plain decode with one query); the HBM-bound verify
// path is the bf16 MFMA kernel over the chunked stores.  Query i of the block sees the
// block's earlier tokens and itself (lucebox post "Laguna XS 2.1 33B on a RTX 3090: 296 tok/s
// peak, 152 tok/s at 256K context", "The model, fast MoE with a drafter in the box": the
// proposals are scored in one batched forward).
//
// Workgroup = (KV head, split of whole 64-key tiles, tile of 64 rows); wave w owns rows
// 16w .. 16w+15.  Per 64-key tile, staged in LDS as f32:
//   S^T [64 keys x 16 rows] = K . Q^T     4 key tiles x (D/4) MFMA 16x16x4
//   online softmax, exact (the running max is updated at every tile)
//   O^T [D x 16 rows]     += V^T . P^T    (D/16) dim tiles x 16 MFMA 16x16x4
// Inside each group of 16 dims the reduction order is permuted so that a lane's four A values
// of four consecutive MFMAs are four consecutive dims (one 16-byte LDS read); the same holds
// for keys in the second product, whose B operand (P^T) is then exactly the accumulator the
// first product left in each lane.
#include "rkv_device.hpp"
#include "rkv_launch.hpp"

namespace rkv {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4v mfma_f32_16x16x4(float a, float b, f32x4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// load 4 consecutive inputs as f32
__device__ __forceinline__ f32x4v load4(const float* p) {
  return *reinterpret_cast<const f32x4v*>(p);
}
__device__ __forceinline__ f32x4v load4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return f32x4v{bf16_bits_to_f32(u.x & 0xffffu), bf16_bits_to_f32(u.x >> 16),
                bf16_bits_to_f32(u.y & 0xffffu), bf16_bits_to_f32(u.y >> 16)};
}
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t* p) { return bf16_bits_to_f32(*p); }

// reductions over the four lanes of a row (lanes n, n+16, n+32, n+48)
__device__ __forceinline__ float row_max4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, typename TIn>
__global__ __launch_bounds__(256) void contig_attn_kernel(ContigArgs a) {
  constexpr int NB = D / 16;     // 16-dim groups
  constexpr int C4 = D / 4;      // 16-byte columns of a K row
  // K [64 keys][D] with the 16-byte column c of key j at c ^ (j & 15); V^T [D][64 keys] with
  // the 16-byte column c of dim d at c ^ (d & 15): the 16 lanes of one read touch 16 rows at
  // one logical column and land in 16 different bank groups.
  __shared__ __attribute__((aligned(16))) float Ks[64 * D];
  __shared__ __attribute__((aligned(16))) float Vt[D * 64];

  const TIn* q = static_cast<const TIn*>(a.q);
  const TIn* k = static_cast<const TIn*>(a.k);
  const TIn* v = static_cast<const TIn*>(a.v);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n16 = lane & 15;
  const int lq = lane >> 4;
  const int g = blockIdx.x % a.n_kv_heads;
  const int s = blockIdx.x / a.n_kv_heads;
  const int G = a.G;
  const int rows = a.q_len * G;
  const int r = blockIdx.y * 64 + w * 16 + n16;
  const bool row_ok = r < rows;
  const int qi = row_ok ? r / G : 0;
  const int hq = g * G + (row_ok ? r % G : 0);
  const int64_t p_i = a.ctx_len - a.q_len + qi;
  const int64_t lo_i = a.window > 0 ? imax64(0, p_i - a.window + 1) : 0;

  // Q^T operand: for MFMA step 4b + t, lane (n16, lq) holds Q[row n16][16b + 4lq + t]
  float qop[4 * NB];
  {
    const TIn* qrow = q + ((int64_t)qi * a.n_q_heads + hq) * D;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const f32x4v x = load4(qrow + 16 * b + 4 * lq);
#pragma unroll
      for (int t = 0; t < 4; ++t) qop[4 * b + t] = row_ok ? x[t] : 0.f;
    }
  }

  const int64_t c_lo = a.c_first + (int64_t)s * a.cps;
  const int64_t c_hi = imin64(c_lo + a.cps, a.c_first + a.n_chunks);
  float m_run = -INFINITY;    // exp2 domain
  float l_run = 0.f;
  f32x4v oacc[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) oacc[t] = f32x4v{0.f, 0.f, 0.f, 0.f};

  for (int64_t c = c_lo; c < c_hi; ++c) {
    const int64_t kbase = c * 64;
    __syncthreads();   // the previous tile's reads are done
#pragma unroll
    for (int u = 0; u < 64 * C4 / 256; ++u) {
      const int e = u * 256 + tid;
      const int key = e / C4, c4 = e % C4;
      const int64_t j = kbase + key;
      f32x4v kx = f32x4v{0.f, 0.f, 0.f, 0.f}, vx = kx;
      if (j < a.ctx_len) {
        const int64_t idx = (j * a.n_kv_heads + g) * D + 4 * c4;
        kx = load4(k + idx);
        vx = load4(v + idx);
      }
      *reinterpret_cast<f32x4v*>(&Ks[key * D + ((c4 ^ (key & 15)) << 2)]) = kx;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int d = 4 * c4 + e2;
        Vt[d * 64 + ((((key >> 2) ^ (d & 15)) << 2) | (key & 3))] = vx[e2];
      }
    }
    __syncthreads();

    // S^T: lane (n16, lq) ends with sacc[tm][i] = S[row n16][key 16tm + 4lq + i]
    f32x4v sacc[4];
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
      sacc[tm] = f32x4v{0.f, 0.f, 0.f, 0.f};
      const int key = 16 * tm + n16;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const f32x4v kv = *reinterpret_cast<const f32x4v*>(&Ks[key * D + (((4 * b + lq) ^ (key & 15)) << 2)]);
#pragma unroll
        for (int t = 0; t < 4; ++t) sacc[tm] = mfma_f32_16x16x4(kv[t], qop[4 * b + t], sacc[tm]);
      }
    }
    // mask (selection: keys past the context hold zeros, not data) and scale
    float mx = -INFINITY;
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t j = kbase + 16 * tm + 4 * lq + i;
        const bool vis = row_ok && j < a.ctx_len && j <= p_i && j >= lo_i;
        sacc[tm][i] = vis ? sacc[tm][i] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sacc[tm][i]);
      }
    }
    const float m_new = fmaxf(m_run, row_max4(mx));
    const float m_use = m_new == -INFINITY ? 0.f : m_new;   // no visible key yet: weights 0
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sacc[tm][i] = exp2f(sacc[tm][i] - m_use);
        lsum += sacc[tm][i];
      }
    }
    l_run = l_run * alpha + row_sum4(lsum);
    // O^T += V^T . P^T, step (tm, i): lane group lq supplies key 16tm + 4lq + i
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      oacc[t] *= alpha;
      const int d = 16 * t + n16;
#pragma unroll
      for (int tm = 0; tm < 4; ++tm) {
        const f32x4v vv = *reinterpret_cast<const f32x4v*>(&Vt[d * 64 + (((4 * tm + lq) ^ (d & 15)) << 2)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[t] = mfma_f32_16x16x4(vv[i], sacc[tm][i], oacc[t]);
      }
    }
  }

  if (!row_ok) return;
  const float l = l_run;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse_nat = l > 0.f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
  float* dst;
  if (a.part_o == nullptr) {
    dst = a.out + ((int64_t)qi * a.n_q_heads + hq) * D;
    if (a.lse != nullptr && lq == 0) a.lse[(int64_t)qi * a.n_q_heads + hq] = lse_nat;
  } else {
    const int64_t prow = ((int64_t)g * a.num_splits + s) * rows + r;
    dst = a.part_o + prow * D;
    if (lq == 0) a.part_lse[prow] = lse_nat;
  }
  // oacc[t][i] = O[row n16][dim 16t + 4lq + i]
#pragma unroll
  for (int t = 0; t < NB; ++t)
    *reinterpret_cast<f32x4v*>(dst + 16 * t + 4 * lq) = oacc[t] * inv;
}

template <int D>
hipError_t launch_d(const ContigArgs& a, hipStream_t stream) {
  const int rows = a.q_len * a.G;
  const dim3 grid(a.n_kv_heads * a.num_splits, (rows + 63) / 64);
  if (a.dtype == 1) return launch_kernel(contig_attn_kernel<D, uint16_t>, grid, dim3(256), a, stream);
  return launch_kernel(contig_attn_kernel<D, float>, grid, dim3(256), a, stream);
}

}  // namespace

hipError_t launch_contig_attn(const ContigArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  return launch_d<64>(a, stream);
}

}  // namespace rkv
