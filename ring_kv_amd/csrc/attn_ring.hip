// Sliding-window verify attention over the position ring in one kernel (lucebox post "Laguna
// XS 2.1 33B on a RTX 3090: 296 tok/s peak, 152 tok/s at 256K context", "3. Ring caches for
// the sliding-window layers": window layers attend a 512-token window through a ring of 2048
// positions, slot = pos mod 2048).
//
// A window layer reads ~1 MB (527 positions per KV head), so it is latency-bound, not
// bandwidth-bound: the kernel is built to put every chunk of the span in flight at once and
// to finish in one launch.  Workgroup = (KV head g, tile of 16 rows); wave w loads whole
// 64-key chunks w, w+8, ... straight from HBM into MFMA operand registers (no LDS staging),
// computes that chunk's online-softmax partial, and the eight partials of a row tile merge
// through LDS into the final output.  The four row tiles of a head read the same chunks, which
// the L2 of their XCD serves after the first.
//
// Operand layouts are those of the chunked split-K kernel: S^T = K Q^T with the key order
// sigma inside pairs of 16-key tiles, then O^T += V^T P^T with P^T straight from the S^T
// accumulators and V^T read as 16 bytes of 8 consecutive keys.
#include "rkv_device.hpp"
#include "rkv_launch.hpp"

namespace rkv {
namespace {

constexpr int kRingWaves = 8;

__device__ __forceinline__ int ring_sigma(int tm, int m) {
  return 32 * (tm >> 1) + 8 * (m >> 2) + 4 * (tm & 1) + (m & 3);
}

__device__ __forceinline__ float ring_row_max4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int D>
__global__ __launch_bounds__(kRingWaves * 64) void ring_attn_kernel(ChunkAttnArgs a) {
  constexpr int KK = D / 32;
  constexpr int TMD = D / 16;
  __shared__ __attribute__((aligned(16))) float xo[kRingWaves][16][D];
  __shared__ float xm[kRingWaves][16];
  __shared__ float xl[kRingWaves][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15;
  const int lq = lane >> 4;
  const int G = a.G;
  const int rows = a.q_len * G;
  const int n_rt = (rows + 15) / 16;
  const int g = blockIdx.x / n_rt;
  const int rt = blockIdx.x % n_rt;

  const int r = rt * 16 + ln;
  const bool row_ok = r < rows;
  const int qi = row_ok ? r / G : 0;
  const int hq = g * G + (row_ok ? r % G : 0);
  const int64_t p_i = a.p0 + qi;
  const int64_t lo_i = a.window > 0 ? imax64(0, p_i - a.window + 1) : 0;
  // visible keys of this row, as absolute positions (stored range included)
  const int64_t vis_lo = imax64(lo_i, a.valid_lo);
  const int64_t vis_hi = row_ok ? imin64(p_i, a.valid_hi - 1) : -1;

  bf16x8 qop[KK];
  {
    const uint16_t* qrow = a.q + ((int64_t)qi * a.n_q_heads + hq) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (row_ok) raw = *reinterpret_cast<const u32x4*>(qrow + kk * 32 + lq * 8);
      qop[kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const bf16x8 ones_col = __builtin_bit_cast(
      bf16x8, ln == 0 ? u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u}
                      : u32x4{0u, 0u, 0u, 0u});
  const float csc = a.scale_log2;

  float m_run = -INFINITY;
  f32x4 oacc[TMD];
  f32x4 lacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < TMD; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t loc = w; loc < a.n_chunks; loc += kRingWaves) {
    const int64_t c = a.c_first + loc;
    const int slot = (int)(c % a.n_slots);
    const int64_t blk = (int64_t)slot * a.n_kv_heads + g;
    const uint16_t* kb = a.k + blk * (64 * D);
    const uint16_t* vb = a.v + blk * (64 * D);
    const int64_t cbase = c * 64;
    // every operand of the chunk is requested before any is used
    u32x4 kraw[4][KK];
    u32x4 vraw[2][TMD];
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kraw[tm][kk] = *reinterpret_cast<const u32x4*>(kb + ring_sigma(tm, ln) * D + (4 * kk + lq) * 8);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int t = 0; t < TMD; ++t)
        vraw[ks][t] = *reinterpret_cast<const u32x4*>(vb + (16 * t + ln) * 64 + (4 * ks + lq) * 8);

    f32x4 sacc[4];
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) sacc[tm] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
        sacc[tm] = mfma_16x16x32(__builtin_bit_cast(bf16x8, kraw[tm][kk]), qop[kk], sacc[tm]);

    const int lo_rel = (int)imax64(-1, imin64(vis_lo - cbase, 64));
    const int hi_rel = (int)imax64(-1, imin64(vis_hi - cbase, 64));
    float mx = -INFINITY;
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kidx = 32 * (tm >> 1) + 8 * lq + 4 * (tm & 1) + i;
        // selection, not arithmetic: a key outside the stored range may hold anything
        if (kidx < lo_rel || kidx > hi_rel) sacc[tm][i] = -INFINITY;
        mx = fmaxf(mx, sacc[tm][i]);
      }
    }
    const float t_max = ring_row_max4(mx) * csc;
    const float m_new = fmaxf(m_run, t_max);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < TMD; ++t) oacc[t] *= alpha;
    lacc *= alpha;

    const bool partial = cbase < a.valid_lo || cbase + 64 > a.valid_hi;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint32_t pw[4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int tm = 2 * ks + hh;
        pw[2 * hh] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sacc[tm][0], csc, -m_use)),
                                 __builtin_amdgcn_exp2f(fmaf(sacc[tm][1], csc, -m_use)));
        pw[2 * hh + 1] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sacc[tm][2], csc, -m_use)),
                                     __builtin_amdgcn_exp2f(fmaf(sacc[tm][3], csc, -m_use)));
      }
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      uint32_t vmask[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
      if (partial) {
        // keys outside the stored range: zero their V so that 0 * (anything) stays 0
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int64_t jj = cbase + 32 * ks + 8 * lq + e;
          if (jj < a.valid_lo || jj >= a.valid_hi) vmask[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        }
      }
#pragma unroll
      for (int t = 0; t < TMD; ++t) {
        u32x4 raw = vraw[ks][t];
        raw[0] &= vmask[0]; raw[1] &= vmask[1]; raw[2] &= vmask[2]; raw[3] &= vmask[3];
        oacc[t] = mfma_16x16x32(__builtin_bit_cast(bf16x8, raw), pb, oacc[t]);
      }
      lacc = mfma_16x16x32(ones_col, pb, lacc);
    }
  }

  // ---- merge the waves' partials of this row tile ------------------------------------------
  const float l = __shfl(lacc[0], ln, kWave);
#pragma unroll
  for (int t = 0; t < TMD; ++t)
    *reinterpret_cast<f32x4*>(&xo[w][ln][16 * t + 4 * lq]) = oacc[t];
  if (lq == 0) {
    xm[w][ln] = m_run;
    xl[w][ln] = l;
  }
  __syncthreads();
  // thread -> (row, 4 consecutive dims); D/4 threads per row, 16 rows
  constexpr int per_row = D / 4;
  if (tid >= 16 * per_row) return;
  const int rr = tid / per_row;
  const int d4 = (tid % per_row) * 4;
  const int r2 = rt * 16 + rr;
  if (r2 >= rows) return;
  const int nw = (int)imin64(kRingWaves, a.n_chunks);
  float M = -INFINITY;
  for (int k = 0; k < nw; ++k) M = fmaxf(M, xm[k][rr]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float L = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < nw; ++k) {
    const float wk = __builtin_amdgcn_exp2f(xm[k][rr] - Mu);
    L += wk * xl[k][rr];
    acc += *reinterpret_cast<const f32x4*>(&xo[k][rr][d4]) * wk;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int qi2 = r2 / G;
  const int h2 = g * G + r2 % G;
  *reinterpret_cast<f32x4*>(a.out + ((int64_t)qi2 * a.n_q_heads + h2) * D + d4) = acc * inv;
  if (a.lse != nullptr && d4 == 0)
    a.lse[(int64_t)qi2 * a.n_q_heads + h2] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_ring_attn(const ChunkAttnArgs& a, hipStream_t stream) {
  const int rows = a.q_len * a.G;
  const int blocks = a.n_kv_heads * ((rows + 15) / 16);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(ring_attn_kernel<128>, dim3(blocks), dim3(kRingWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL(ring_attn_kernel<64>, dim3(blocks), dim3(kRingWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rkv
