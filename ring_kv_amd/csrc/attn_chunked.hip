// Verify-block attention over a chunked KV store: the paged pool of 64-token chunks
// (lucebox post "Laguna XS 2.1 33B on a RTX 3090: 296 tok/s peak, 152 tok/s at 256K
// context", "Three optimizations", item 1) and the sliding-window position ring (same
// post, "3. Ring caches for the sliding-window layers").  The ring is a store of
// ring_size/64 chunk slots in which logical chunk c sits in slot c mod (ring_size/64), so
// both stores go through one kernel that differs only in the chunk -> slot rule.
//
// One workgroup = one KV head g and one range of whole chunks (a split).  Its rows are the
// q_len * G (query, query-head) pairs that read head g; wave w owns rows 16w .. 16w+15.
// Per chunk, for every wave:
//   S^T [64 keys x 16 rows] = K [64 x D] . Q^T       4 x (D/32) MFMA 16x16x32 bf16
//   online softmax over the chunk's 64 keys per row   (f32, exp2 domain)
//   O^T [D x 16 rows]     += V^T [D x 64] . P^T       (D/16) x 2 MFMA
// Computing S transposed leaves each lane with 16 scores of ONE row, which is exactly the
// B-operand layout of P^T for the second product: no LDS round trip for P.  Within a pair
// of 16-key tiles the key order is permuted (sigma below) so that each lane's 8 P values
// are 8 consecutive keys, which the dimension-major V chunk supplies as one 16-byte read.
//
// Memory path: K and V chunks are streamed from HBM with 16-byte loads (a wave reads 1 KiB
// contiguous per instruction), two chunks ahead of the compute, staged in registers and
// written into double-buffered, XOR-swizzled LDS tiles that all waves read.
#include "rkv_device.hpp"
#include "rkv_launch.hpp"

namespace rkv {

namespace {

// S^T row m of 16-key tile tm -> key within the chunk.  Lane group q of the C layout holds
// rows 4q..4q+3 of each tile; tiles 2ks and 2ks+1 together give that lane keys
// 32ks + 8q + 0..7.
__device__ __forceinline__ int sigma(int tm, int m) {
  return 32 * (tm >> 1) + 8 * (m >> 2) + 4 * (tm & 1) + (m & 3);
}

__device__ __forceinline__ int swz_k(int key) { return (key & 3) | (((key >> 3) & 1) << 2); }
__device__ __forceinline__ int swz_v(int d) { return d & 7; }

constexpr int kPtCap = 512;   // page-table entries kept in LDS (a power of two, >= 512)

template <int D>
struct Tile {
  static constexpr int kRow = D / 8;           // 16-byte pieces per K row
  static constexpr int kPieces = 64 * kRow;    // K pieces per chunk
  static constexpr int vPieces = D * 8;        // V pieces per chunk (D rows of 64 keys)
  static constexpr int elems = 2 * 64 * D;     // bf16 elements per LDS buffer
  // LDS offsets in bf16 elements
  __device__ static __forceinline__ int k_off(int key, int piece) {
    return key * D + ((piece ^ swz_k(key)) << 3);
  }
  __device__ static __forceinline__ int v_off(int d, int piece) {
    return 64 * D + d * 64 + ((piece ^ swz_v(d)) << 3);
  }
};

// Direct HBM -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4): lane i of
// the wave writes LDS bytes [lds_base + 16 i, +16).  Issued from inline assembly so that the
// compiler neither reorders these loads nor inserts its own (all-draining) waits for them;
// the kernel waits on the vector-memory counter itself.
__device__ __forceinline__ void dma16(uint32_t lds_base, const void* gbase, uint32_t goff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_base), "v"(goff), "s"(gbase) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// PAGED: slots come from the page table; otherwise the store is a ring (slot = c mod n_slots).
template <int D, int NW, int NBUF, bool PAGED>
__global__ __launch_bounds__(NW * 64)
void chunk_attn_kernel(ChunkAttnArgs a) {
  using T = Tile<D>;
  constexpr int NT = NW * 64;
  constexpr int LPC = (T::kPieces + T::vPieces) / NT;   // 16-byte loads per chunk per thread
  static_assert((T::kPieces + T::vPieces) % NT == 0, "pieces must divide evenly");
  static_assert(T::kPieces % 64 == 0, "a wave's load must fall in one tile");
  constexpr int PF = NBUF - 1;                           // chunks in flight ahead of compute
  static_assert(PF >= 1 && (PF - 1) * LPC < 64, "vmcnt range");
  constexpr int KK = D / 32;
  constexpr int TMD = D / 16;
  constexpr uint32_t kBufBytes = T::elems * 2;

  __shared__ __attribute__((aligned(16))) uint16_t lds[NBUF][T::elems];
  __shared__ int pt_lds[kPtCap];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15;
  const int lq = lane >> 4;

  const int b = xcd_block(blockIdx.x, gridDim.x);
  const int g = b % a.n_kv_heads;
  const int s = b / a.n_kv_heads;
  const int G = a.G;
  const int rows = a.q_len * G;

  const int64_t c_lo = a.c_first + (int64_t)s * a.cps;
  const int64_t c_end = a.c_first + a.n_chunks;
  const int nloc = (int)imax64(0, imin64((int64_t)a.cps, c_end - c_lo));

  // ---- this lane's query row ---------------------------------------------------------
  const int r = w * 16 + ln;
  const bool row_ok = r < rows;
  const int qi = row_ok ? r / G : 0;
  const int hq = g * G + (row_ok ? r % G : 0);
  const int64_t p_i = a.p0 + qi;
  const int64_t lo_i = a.window > 0 ? imax64(0, p_i - a.window + 1) : 0;
  const bool wave_active = w * 16 < rows;
  const int64_t p_first = a.p0;
  const int64_t p_last = a.p0 + a.q_len - 1;
  const int64_t lo_last = a.window > 0 ? imax64(0, p_last - a.window + 1) : 0;

  // Q^T operand of S^T = K Q^T: lane (ln, lq) holds row ln's dims kk*32 + 8*lq .. +7
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

  // ---- page-table slice in LDS: entry for local chunk loc at pt_lds[loc % kPtCap] -----
  // Filled once for the first kPtCap chunks; splits longer than that refresh one half of the
  // slice at a time, 128 chunks before it is needed.
  constexpr bool paged = PAGED;
  if (paged) {
    for (int e = tid; e < kPtCap && e < nloc; e += NT) pt_lds[e] = a.pt[c_lo + e];
  }
  // Q and the table slice are in registers / LDS before any chunk load is issued, so the
  // compiler's own waits for them never cover a chunk load.
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(qop[kk]));
  lds_barrier();

  // ring: slot = logical chunk mod n_slots; a ring span covers at most n_slots + 1 chunks
  const int ring_base = paged ? 0 : (int)(c_lo % a.n_slots);
  auto slot_of = [&](int loc) -> int {
    if (!paged) {
      int t = ring_base + loc;
      t -= t >= a.n_slots ? a.n_slots : 0;
      t -= t >= a.n_slots ? a.n_slots : 0;
      return t;
    }
    return __builtin_amdgcn_readfirstlane(pt_lds[loc & (kPtCap - 1)]);
  };
  auto maybe_refresh_table = [&](int loc) {
    // at loc = 256k + 128 (k >= 1) load local chunks [256(k+1), 256(k+2)) into half (k+1)&1,
    // which last held chunks [256(k-1), 256k), all issued by now
    if (!paged || nloc <= kPtCap || (loc & 255) != 128 || loc < 256) return;
    const int base = ((loc >> 8) + 1) << 8;
    if (base >= nloc) return;
    for (int e = tid; e < 256; e += NT)
      if (base + e < nloc) pt_lds[(base + e) & (kPtCap - 1)] = a.pt[c_lo + base + e];
  };

  const uint32_t lds_base = (uint32_t)(uintptr_t)&lds[0][0];
  // Chunk loc -> LDS buffer loc % NBUF.  LDS piece P of a buffer (P = u*NT + 64w + lane) holds
  // global piece P with the XOR swizzle undone, so every wave instruction still reads 1 KiB of
  // contiguous HBM.  An out-of-range slot loads slot 0 instead (the chunk is skipped in compute)
  // so that every thread always has exactly LPC loads per chunk outstanding.
  auto issue = [&](int loc) {
    int slot = slot_of(loc);
    if ((unsigned)slot >= (unsigned)a.n_slots) slot = 0;
    const int64_t blk = (int64_t)slot * a.n_kv_heads + g;
    const uint16_t* kb = a.k + blk * (64 * D);
    const uint16_t* vb = a.v + blk * (64 * D);
    const uint32_t lb = lds_base + (uint32_t)(loc % NBUF) * kBufBytes;
#pragma unroll
    for (int u = 0; u < LPC; ++u) {
      const int pw = u * NT + w * 64;                     // first piece of this wave's load
      const int P = pw + lane;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(lb + (uint32_t)pw * 16u);
      if (pw < T::kPieces) {
        const int key = P / T::kRow, phys = P % T::kRow;
        dma16(m0, kb, (uint32_t)(key * T::kRow + (phys ^ swz_k(key))) * 16u);
      } else {
        const int vp = P - T::kPieces;
        const int d = vp >> 3, phys = vp & 7;
        dma16(m0, vb, (uint32_t)(d * 8 + (phys ^ swz_v(d))) * 16u);
      }
    }
  };

  // ---- running softmax state ---------------------------------------------------------
  float m_run = -INFINITY;   // exp2-domain running max of this lane's row
  float l_run = 0.f;         // this lane's share of the row sum (reduced at the end)
  f32x4 oacc[TMD];
#pragma unroll
  for (int t = 0; t < TMD; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint16_t* buf, int loc) {
    if (!wave_active) return;
    if ((unsigned)slot_of(loc) >= (unsigned)a.n_slots) return;   // no slot: adds nothing
    const int64_t cbase = (c_lo + loc) * 64;
    const bool partial = cbase < a.valid_lo || cbase + 64 > a.valid_hi;
    const bool edge = (cbase + 63 > p_first) || (cbase < lo_last) || partial;
    // four independent 16-key tiles per k-step keep the matrix pipe busy
    f32x4 sacc[4];
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) sacc[tm] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8 ka[4];
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
        ka[tm] = *reinterpret_cast<const bf16x8*>(buf + T::k_off(sigma(tm, ln), 4 * kk + lq));
#pragma unroll
      for (int tm = 0; tm < 4; ++tm) sacc[tm] = mfma_16x16x32(ka[tm], qop[kk], sacc[tm]);
    }
    float sc[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float t = sacc[tm][i] * a.scale_log2;
        if (edge) {
          // selection, not arithmetic: a key outside the stored range may hold anything
          const int64_t j = cbase + 32 * (tm >> 1) + 8 * lq + 4 * (tm & 1) + i;
          if (!row_ok || j < lo_i || j > p_i) t = -INFINITY;
        }
        sc[tm][i] = t;
        mx = fmaxf(mx, t);
      }
    }
    mx = fmaxf(mx, wave_xor(mx, 16));
    mx = fmaxf(mx, wave_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    uint32_t pw[2][4];   // P^T operand words for ks = 0, 1
    float lsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int tm = 2 * ks + hh;
        const float p0 = __builtin_amdgcn_exp2f(sc[tm][0] - m_use);
        const float p1 = __builtin_amdgcn_exp2f(sc[tm][1] - m_use);
        const float p2 = __builtin_amdgcn_exp2f(sc[tm][2] - m_use);
        const float p3 = __builtin_amdgcn_exp2f(sc[tm][3] - m_use);
        const uint32_t w01 = pack_bf16x2(p0, p1);
        const uint32_t w23 = pack_bf16x2(p2, p3);
        pw[ks][2 * hh] = w01;
        pw[ks][2 * hh + 1] = w23;
        // the row sum uses the same rounded weights the PV product sees
        lsum += __uint_as_float(w01 << 16) + __uint_as_float(w01 & 0xffff0000u) +
                __uint_as_float(w23 << 16) + __uint_as_float(w23 & 0xffff0000u);
      }
    }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int t = 0; t < TMD; ++t) oacc[t] *= alpha;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pw[ks][0], pw[ks][1], pw[ks][2], pw[ks][3]});
      // keys outside the stored range: zero their V so that 0 * (anything) stays 0
      uint32_t vmask[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
      if (partial) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int64_t j = cbase + 32 * ks + 8 * lq + e;
          if (j < a.valid_lo || j >= a.valid_hi) vmask[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        }
      }
#pragma unroll
      for (int t = 0; t < TMD; ++t) {
        u32x4 raw = *reinterpret_cast<const u32x4*>(buf + T::v_off(16 * t + ln, 4 * ks + lq));
        if (partial) {
          raw[0] &= vmask[0]; raw[1] &= vmask[1]; raw[2] &= vmask[2]; raw[3] &= vmask[3];
        }
        oacc[t] = mfma_16x16x32(__builtin_bit_cast(bf16x8, raw), pb, oacc[t]);
      }
    }
  };

  // ---- pipeline: PF chunks in flight while one is computed -----------------------------
#pragma unroll
  for (int k = 0; k < PF; ++k)
    if (k < nloc) issue(k);

  for (int loc = 0; loc < nloc; ++loc) {
    // chunks issued after this one: min(PF-1, nloc-1-loc); wait until only they are in flight
    const int ahead = nloc - 1 - loc;
    if (ahead >= PF - 1) wait_vmcnt<(PF - 1) * LPC>();
    else if (PF >= 3 && ahead == 1) wait_vmcnt<LPC>();
    else wait_vmcnt<0>();
    lds_barrier();
    // refill the buffer computed in the previous step (every wave is past it now)
    maybe_refresh_table(loc + PF);
    if (loc + PF < nloc) issue(loc + PF);
    compute(&lds[loc % NBUF][0], loc);
  }

  // ---- epilogue ------------------------------------------------------------------------
  if (!wave_active) return;
  float l = l_run;
  l += wave_xor(l, 16);
  l += wave_xor(l, 32);
  if (!row_ok) return;
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
#pragma unroll
  for (int t = 0; t < TMD; ++t) {
    f32x4 o = oacc[t] * inv;
    *reinterpret_cast<f32x4*>(dst + 16 * t + 4 * lq) = o;
  }
}

template <int D, int NW>
hipError_t launch_t(const ChunkAttnArgs& a, hipStream_t stream) {
  const int blocks = a.n_kv_heads * a.num_splits;
  // four LDS chunk buffers (3 chunks in flight); D = 128 uses 128 KiB + the table slice
  if (a.pt != nullptr)
    hipLaunchKernelGGL((chunk_attn_kernel<D, NW, 4, true>), dim3(blocks), dim3(NW * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((chunk_attn_kernel<D, NW, 4, false>), dim3(blocks), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const ChunkAttnArgs& a, hipStream_t stream) {
  const int rows = a.q_len * a.G;
  if (rows <= 64) return launch_t<D, 4>(a, stream);
  if (rows <= 128) return launch_t<D, 8>(a, stream);
  return launch_t<D, 16>(a, stream);
}

}  // namespace

hipError_t launch_chunk_attn(const ChunkAttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  return launch_d<64>(a, stream);
}

}  // namespace rkv
