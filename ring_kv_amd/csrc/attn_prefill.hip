// Attention of a long query block (batched prefill: hundreds to thousands of queries) over a
// chunked KV store: the paged pool of 64-token chunks (lucebox post "Laguna XS 2.1 33B on a
// RTX 3090: 296 tok/s peak, 152 tok/s at 256K context", "Three optimizations", item 1) and the
// sliding-window position ring (same post, "3. Ring caches for the sliding-window layers"; its
// "TL;DR" runs prefill as pooled batches plus ring attention).  Same arguments, definition and
// partial format as the verify-block kernel; what differs is the balance of work.  A 16-query
// verify block is bound by streaming the KV from HBM; a 1024-query block does 64 times the
// arithmetic per key and is bound by the matrix cores, so the tiling favours reuse of every
// K/V element staged in LDS:
//
//   workgroup = one KV head g, one split (range of whole chunks), one tile of 32*NRG rows in 8
//   waves; each wave owns 32 rows and computes, per 64-key chunk (KS = 1) or per 32-key half of
//   it (KS = 2: two waves per row group, one per half),
//     S^T [64 keys x 32 rows] = K [64 x D] . Q^T          2 x (D/16) MFMA 32x32x16 bf16
//     online softmax of each row over the chunk's keys  (f32, exp2 domain)
//     O^T [D x 32 rows]     += V^T [D x 64] . P^T         (D/32) x 4 MFMA 32x32x16 bf16
//   (half of each with KS = 2, whose two halves merge their softmax states at the end).
//   256-row tiles give every K/V element staged in LDS the most reuse; 128-row tiles (KS = 2)
//   double the workgroups of a block whose 256-row grid leaves most of the chip idle, and
//   64-row tiles (two row groups, KS = 2) quadruple them where that grid still fits one round
//   (a block over the ring, where each tile sees only its window and is not split).
//
// S is computed transposed so that each lane ends with 16 scores of ONE row per 32-key tile,
// which after a fixed permutation of the keys (rho below) is exactly the B operand of P^T for
// the second product: P never goes through LDS.  Q stays in registers for the whole split.
//
// A workgroup only visits the chunks its rows can see (its tile's causal end and, for a window,
// its first query's window start), so a split of the key range may leave a tile nothing to do:
// its partial is then empty (lse -inf), which the merge gives no weight.
#include "rkv_device.hpp"
#include "rkv_launch.hpp"

#include <type_traits>

namespace rkv {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// 32x32x16 bf16 MFMA: lane l supplies row (l & 31) of A and column (l & 31) of B, each as 8
// k-values of k-group (l >> 5); C lane l holds column (l & 31), rows 8*(v/4) + 4*(l>>5) + v%4
// for its 16 items v.
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// S^T row i of 32-key tile kt -> key within the chunk: bits 2 and 3 of i swapped.  Lane half h
// then holds, in items 8b .. 8b+7 of tile kt, the keys 16*(2kt+b) + 8h + 0..7: for every
// 16-key block of the PV product, the 8 consecutive keys its B operand wants from that lane.
__device__ __forceinline__ int rho(int kt, int i) {
  return 32 * kt + ((i & 0x13) | ((i & 4) << 1) | ((i & 8) >> 1));
}

// XOR swizzles of the 16-byte pieces of an LDS row.  A K operand read touches 32 keys rho(kt, m)
// at one piece; the swizzle is a function of the key's low bits chosen so that every group of 8
// lanes hits 8 distinct 16-byte slots of a 128-byte bank line and every group of 16 lanes 16
// distinct slots of a 256-byte line.  V^T reads touch 32 consecutive dimension rows at one piece.
template <int D>
__device__ __forceinline__ int swz_k(int key) {
  return D == 128 ? ((key & 3) | ((key >> 1) & 4) | ((key << 1) & 8))
                  : (((key ^ (key >> 2)) & 1) | (key & 2) | ((key >> 1) & 4));
}
__device__ __forceinline__ int swz_v(int d) { return ((d >> 1) & 7) ^ ((d & 1) << 2); }

// Lazy rescaling: a row keeps its reference max while its weights stay below 2^8, so the
// accumulators are rescaled only rarely; a row without a reference yet keeps 0 as long as its
// weights stay above 2^-8 (well inside f32 and bf16 range).
constexpr float kSlackHi = 256.0f;
constexpr float kSlackLo = 1.0f / 256.0f;

__device__ __forceinline__ int rel_pos(int64_t x, int64_t base) {
  return (int)imax64(-(int64_t(1) << 29), imin64(x - base, int64_t(1) << 29));
}

// the other lane of this lane's row (lane ^ 32) and this lane's value, combined by max / sum
__device__ __forceinline__ float pair_max(float v) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D>
struct PTile {
  static constexpr int kRow = D / 8;            // 16-byte pieces per K row
  static constexpr int kPieces = 64 * kRow;     // K pieces per chunk
  static constexpr int vPieces = D * 8;         // V pieces per chunk
  static constexpr int elems = 2 * 64 * D;      // bf16 elements per LDS tile
  __device__ static __forceinline__ int k_off(int key, int piece) {
    return key * D + ((piece ^ swz_k<D>(key)) << 3);
  }
  __device__ static __forceinline__ int v_off(int d, int piece) {
    return 64 * D + d * 64 + ((piece ^ swz_v(d)) << 3);
  }
};

template <int D, int NRG, int KS, bool PAGED>
__global__ __launch_bounds__(NRG * KS * 64, 2)
void prefill_attn_kernel(ChunkAttnArgs a) {
  using T = PTile<D>;
  constexpr int NW = NRG * KS;
  constexpr int NT = NW * 64;
  constexpr int ROWS = 32 * NRG;
  constexpr int NKT = KS == 2 ? 1 : 2;    // 32-key tiles per chunk computed by one wave
  constexpr int LPC = (T::kPieces + T::vPieces) / NT;   // 16-byte loads per chunk per thread
  static_assert((T::kPieces + T::vPieces) % NT == 0 && T::kPieces % NT == 0, "piece split");
  constexpr int KK = D / 16;    // 16-dim steps of S^T
  constexpr int DT = D / 32;    // 32-dim tiles of O^T

  __shared__ __attribute__((aligned(16))) uint16_t lds[2][T::elems];
  __shared__ float xstate[KS == 2 ? NRG * 3 * 64 : 1];   // key half 1's m, l_run, l_rnd per lane

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = w % NRG;                 // row group: rows 32rg .. 32rg+31 of the tile
  const int kh = w / NRG;                 // key half (KS = 2): keys 32kh .. 32kh+31 of a chunk
  const int n = lane & 31;
  const int h = lane >> 5;

  // ---- work item: (KV head, split, row tile), consecutive tiles of one (head, split) on one XCD
  const int n_tiles = gridDim.x / (a.n_kv_heads * a.num_splits);
  const int b = xcd_block(blockIdx.x, gridDim.x);
  const int tile = b % n_tiles;
  const int gs = b / n_tiles;
  const int g = gs % a.n_kv_heads;
  const int s = gs / a.n_kv_heads;
  const int G = a.G;
  const int rows = a.q_len * G;
  const int row0 = tile * ROWS;

  // ---- the chunks this tile can see within its split ----------------------------------------
  const int64_t tq0 = row0 / G;
  const int64_t tq1 = (int64_t)(min(row0 + ROWS, rows) - 1) / G;
  const int64_t p_first64 = a.p0 + tq0;                      // earliest query of the tile
  const int64_t p_last64 = a.p0 + tq1;
  const int64_t lo_first64 = a.window > 0 ? imax64(0, p_first64 - a.window + 1) : 0;
  const int64_t lo_last64 = a.window > 0 ? imax64(0, p_last64 - a.window + 1) : 0;
  const int64_t s_lo = a.c_first + (int64_t)s * a.cps;
  const int64_t s_hi = imin64(s_lo + a.cps, a.c_first + a.n_chunks);
  const int64_t c_from = imax64(s_lo, imax64(lo_first64, a.valid_lo) / 64);
  const int64_t c_to = imin64(s_hi, imin64(p_last64, a.valid_hi - 1) / 64 + 1);
  const int nloc = (int)imax64(0, c_to - c_from);

  // ---- this lane's row -------------------------------------------------------------------------
  const int r = row0 + 32 * rg + n;
  const bool row_ok = r < rows;
  const int qi = row_ok ? r / G : 0;
  const int hq = g * G + (row_ok ? r % G : 0);
  const int64_t pbase = c_from * 64;
  const int64_t p_i64 = a.p0 + qi;
  const int p_i = rel_pos(p_i64, pbase);
  const int lo_i = rel_pos(a.window > 0 ? imax64(0, p_i64 - a.window + 1) : 0, pbase);
  const int vlo = rel_pos(a.valid_lo, pbase);
  const int vhi = rel_pos(a.valid_hi, pbase);

  // ---- slots ------------------------------------------------------------------------------------
  constexpr bool paged = PAGED;
  const int ring_base = paged ? 0 : (int)(c_from % a.n_slots);
  // The slot of local chunk loc (loc < nloc), or -1 when the table points outside the pool, in
  // two halves: fetch() starts the read, slot() turns its result into the slot.  The table is
  // read with a vector load (through an offset the compiler cannot see to be uniform) one step
  // before the slot is needed: a scalar load would share its wait counter with the LDS reads
  // and stall the first of them in every step.
  int vzero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
  auto fetch = [&](int loc) __attribute__((always_inline)) -> int {
    if (!paged) return loc;
    return a.pt[c_from + min(loc, nloc - 1) + vzero];
  };
  auto slot = [&](int fetched) __attribute__((always_inline)) -> int {
    if (!paged) {
      int t = ring_base + fetched % a.n_slots;
      return t >= a.n_slots ? t - a.n_slots : t;
    }
    const int v = __builtin_amdgcn_readfirstlane(fetched);
    return (unsigned)v < (unsigned)a.n_slots ? v : -1;
  };
  // every table entry of the range in the pool?  (else every chunk takes the masking path)
  bool table_ok = true;
  if (paged) {
    bool bad = false;
    for (int e = tid; e < nloc; e += NT) bad |= (unsigned)a.pt[c_from + e] >= (unsigned)a.n_slots;
    table_ok = !__syncthreads_or(bad);
  }

  // ---- register stage: chunk loads, 1 KiB of contiguous HBM per wave instruction -------------
  u32x4 stg[LPC];
  auto issue = [&](int slot) __attribute__((always_inline)) {
    const int sl = slot >= 0 ? slot : 0;                       // no slot: filler, never used
    const int64_t blk = (int64_t)sl * a.n_kv_heads + g;
    const uint16_t* kb = a.k + blk * (64 * D);
    const uint16_t* vb = a.v + blk * (64 * D);
#pragma unroll
    for (int u = 0; u < LPC; ++u) {
      const int P = u * NT + tid;
      const uint16_t* src = (u * NT < T::kPieces) ? kb + P * 8 : vb + (P - T::kPieces) * 8;
      stg[u] = *reinterpret_cast<const u32x4*>(src);
    }
  };
  auto commit = [&](uint16_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < LPC; ++u) {
      const int P = u * NT + tid;
      int off;
      if (u * NT < T::kPieces) {
        off = T::k_off(P / T::kRow, P % T::kRow);
      } else {
        const int vp = P - T::kPieces;
        off = T::v_off(vp >> 3, vp & 7);
      }
      *reinterpret_cast<u32x4*>(buf + off) = stg[u];
    }
  };

  // ---- Q^T operand: lane (n, h) holds row n's dims 16kk + 8h .. +7 -------------------------------
  bf16x8 qop[KK];
  {
    const uint16_t* qrow = a.q + ((int64_t)qi * a.n_q_heads + hq) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + kk * 16 + h * 8);
      if (!row_ok) raw = u32x4{0u, 0u, 0u, 0u};
      qop[kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // ---- running state: m_run (exp2 domain, shared by the row's two lanes), this lane's shares of
  // the row sums, O^T accumulators ------------------------------------------------------------
  float m_run = -INFINITY;
  float l_run = 0.f;      // sum of the f32 weights
  float l_rnd = 0.f;      // sum of the same weights rounded to bf16
  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[t][v] = 0.f;
  const float csc = a.scale_log2;

  // Per chunk (KS = 1): S^T of both 32-key tiles first, then tile by tile the softmax and its
  // half of the PV product.  The order lets the matrix core run tile 1's QK products while the
  // vector unit works on tile 0's scores, and tile 0's PV products while it works on tile 1's.
  // With KS = 2 a wave computes only tile kh and the two waves of a SIMD overlap instead.
  auto compute = [&](const uint16_t* buf, int loc, bool ok, auto edge_tag) __attribute__((always_inline)) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const int cbase = loc * 64;
    f32x16 sacc[NKT];
#pragma unroll
    for (int j = 0; j < NKT; ++j) {
      const int kt = KS == 2 ? kh : j;
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[j][v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(buf + T::k_off(rho(kt, n), 2 * kk + h));
        sacc[j] = mfma_32x32x16(ka, qop[kk], sacc[j]);
      }
    }
    // visible keys of this row relative to the chunk, and the V words of keys without a stored
    // row or slot (zeroed, so that 0 * (anything) = 0)
    int vis_lo = 0, vis_hi = 63;
    bool vzero = false;
    if constexpr (EDGE) {
      vis_lo = max(-1, min(max(lo_i, vlo) - cbase, 64));
      vis_hi = (row_ok && ok) ? max(-1, min(min(p_i, vhi - 1) - cbase, 64)) : -1;
      vzero = !ok || cbase < vlo || cbase + 64 > vhi;
    }
#pragma unroll
    for (int j = 0; j < NKT; ++j) {
      const int kt = KS == 2 ? kh : j;
      // item v of tile kt is key 32kt + 16(v/8) + 8h + v%8 of the chunk
      if constexpr (EDGE) {
        // key - 32kt - 8h is a compile-time constant per item: compare it with the bounds
        // shifted by 32kt + 8h
        const int lo8 = vis_lo - 32 * kt - 8 * h, hi8 = vis_hi - 32 * kt - 8 * h;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kc = 16 * (v >> 3) + (v & 7);
          if (kc < lo8 || kc > hi8) sacc[j][v] = -INFINITY;    // select, not arithmetic
        }
      }
      // Weights against the row's current reference m_use (0 before the row has one); the max
      // is taken over the weights, which the compiler knows are never NaN, rather than over the
      // raw scores.  A row whose weights leave [2^-S, 2^S] while it has no reference yet, or
      // pass 2^S, takes the rare path: reference = the tile's true max, accumulators rescaled,
      // weights recomputed.
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      float pv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) pv[v] = __builtin_amdgcn_exp2f(fmaf(sacc[j][v], csc, -m_use));
      float pm = pv[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) pm = fmaxf(pm, pv[v]);
      pm = pair_max(pm);
      const bool grow = pm > kSlackHi || (m_run == -INFINITY && pm < kSlackLo);
      if (__builtin_amdgcn_ballot_w64(grow)) {
        // the empty volatile asm keeps the compiler from executing this path unconditionally
        asm volatile("" ::);
        float mx = sacc[j][0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sacc[j][v]);
        const float t_max = pair_max(mx) * csc;
        const float m_new = (grow && t_max != -INFINITY) ? t_max : m_use;
        const float alpha = (grow && m_run != -INFINITY) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
        l_run *= alpha;
        l_rnd *= alpha;
#pragma unroll
        for (int v = 0; v < 16; ++v) pv[v] = __builtin_amdgcn_exp2f(fmaf(sacc[j][v], csc, -m_new));
        m_run = (grow && t_max == -INFINITY) ? m_run : m_new;
      } else {
        m_run = m_use;
      }
      // P^T operand of 16-key block kb = 2kt + hb: items 8hb .. 8hb+7 of the tile.  Two row sums:
      // of the f32 weights (for the lse) and of the bf16 weights the PV product multiplies (to
      // normalise the output, so that a row dominated by one key gets exactly that key's V)
      float lsum = 0.f, lsum_r = 0.f;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        uint32_t wds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wds[e] = pack_bf16x2(pv[8 * hb + 2 * e], pv[8 * hb + 2 * e + 1]);
          lsum += pv[8 * hb + 2 * e] + pv[8 * hb + 2 * e + 1];
          lsum_r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wds[e]), kOnes2,
                                                   lsum_r, false);
        }
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{wds[0], wds[1], wds[2], wds[3]});
        const int kb = 2 * kt + hb;
        uint32_t vmask[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
        if constexpr (EDGE) {
          if (vzero) {
            // key cbase + 16kb + 8h + e is stored iff 16hb + e lies in [slo, shi)
            const int slo = ok ? vlo - cbase - 32 * kt - 8 * h : 64;
            const int shi = vhi - cbase - 32 * kt - 8 * h;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int kc = 16 * hb + e;
              if (kc < slo || kc >= shi) vmask[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
            }
          }
        }
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          u32x4 raw = *reinterpret_cast<const u32x4*>(buf + T::v_off(32 * t + n, 2 * kb + h));
          if constexpr (EDGE) {
            raw[0] &= vmask[0]; raw[1] &= vmask[1]; raw[2] &= vmask[2]; raw[3] &= vmask[3];
          }
          oacc[t] = mfma_32x32x16(__builtin_bit_cast(bf16x8, raw), pb, oacc[t]);
        }
      }
      l_run += lsum;
      l_rnd += lsum_r;
    }
  };

  // ---- pipeline: chunk loc + 1 in registers while chunk loc is computed ------------------------
  // Step loc: barrier (every wave is done with chunk loc - 1, and chunk loc's tile is written);
  // write chunk loc + 1 from the stage into the other tile; load chunk loc + 2 into the stage;
  // compute chunk loc.  Loads past the range read slot 0 and are never computed.
  if (nloc > 0) {
    int sl_cur = slot(fetch(0));
    int sl_nxt = nloc > 1 ? slot(fetch(1)) : -1;
    int f_far = fetch(2);                  // slot of chunk loc + 2, still to be converted
    issue(sl_cur);
    commit(&lds[0][0]);
    issue(sl_nxt);

    auto step = [&](int loc, auto edge_tag) __attribute__((always_inline)) {
      lds_barrier();
      commit(&lds[(loc + 1) & 1][0]);
      const int sl_far = loc + 2 < nloc ? slot(f_far) : -1;
      issue(sl_far);
      f_far = fetch(loc + 3);
      compute(&lds[loc & 1][0], loc, sl_cur >= 0, edge_tag);
      sl_cur = sl_nxt;
      sl_nxt = sl_far;
    };
    // interior chunks [ca, cb): after every row's window start and the stored range's start,
    // ending at or before the tile's first query and the stored range's end
    int ca = nloc, cb = nloc;
    if (table_ok) {
      const int lead = max(max(rel_pos(lo_last64, pbase), vlo), 0);
      ca = min((lead + 63) / 64, nloc);
      const int end = max(min(rel_pos(p_first64, pbase) + 1, vhi), 0) / 64;
      cb = max(ca, min(end, nloc));
    }
    int loc = 0;
    for (; loc < ca; ++loc) step(loc, std::true_type{});
    for (; loc < cb; ++loc) step(loc, std::false_type{});
    for (; loc < nloc; ++loc) step(loc, std::true_type{});
  }

  // ---- epilogue ---------------------------------------------------------------------------------
  if constexpr (KS == 2) {
    // Key half 1 hands its state to key half 0 through the idle LDS tiles (32 rows x D floats per
    // row group: exactly the two tiles); row n's 16-byte pieces are XOR-swizzled by n so that a
    // wave's 32 rows spread over all banks.  Both states are relative to their own reference
    // max; a half that saw no visible key has m = -inf and weighs nothing.
    static_assert(NRG * 32 * D * 4 <= 2 * T::elems * 2, "exchange fits the tiles");
    float* xo = reinterpret_cast<float*>(&lds[0][0]);
    auto xo_off = [&](int t, int j) __attribute__((always_inline)) {
      const int piece = 8 * t + 2 * j + h;                 // dims 32t + 8j + 4h .. +3
      return (rg * 32 + n) * D + ((piece ^ (n & (D / 4 - 1))) << 2);
    };
    lds_barrier();                                         // every wave is done with the tiles
    if (kh == 1) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4*>(&xo[xo_off(t, j)]) =
              f32x4{oacc[t][4 * j], oacc[t][4 * j + 1], oacc[t][4 * j + 2], oacc[t][4 * j + 3]};
      xstate[(rg * 3 + 0) * 64 + lane] = m_run;
      xstate[(rg * 3 + 1) * 64 + lane] = l_run;
      xstate[(rg * 3 + 2) * 64 + lane] = l_rnd;
    }
    lds_barrier();
    if (kh == 1) return;
    const float m1 = xstate[(rg * 3 + 0) * 64 + lane];
    const float M = fmaxf(m_run, m1);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float a0 = __builtin_amdgcn_exp2f(m_run - Mu);    // -inf -> 0
    const float a1 = __builtin_amdgcn_exp2f(m1 - Mu);
    l_run = l_run * a0 + xstate[(rg * 3 + 1) * 64 + lane] * a1;
    l_rnd = l_rnd * a0 + xstate[(rg * 3 + 2) * 64 + lane] * a1;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(&xo[xo_off(t, j)]);
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[t][4 * j + e] = oacc[t][4 * j + e] * a0 + o1[e] * a1;
      }
    m_run = M;
  }
  if (!row_ok) return;
  const float l = pair_sum(l_run);
  const float lr = pair_sum(l_rnd);
  const float inv = lr > 0.f ? 1.f / lr : 0.f;
  const float lse_nat = l > 0.f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
  float* dst;
  if (a.part_o == nullptr) {
    dst = a.out + ((int64_t)qi * a.n_q_heads + hq) * D;
    if (a.lse != nullptr && h == 0) a.lse[(int64_t)qi * a.n_q_heads + hq] = lse_nat;
  } else {
    const int64_t prow = ((int64_t)g * a.num_splits + s) * rows + r;
    dst = a.part_o + prow * D;
    if (h == 0) a.part_lse[prow] = lse_nat;
  }
  // item v of dim tile t is dimension 32t + 8(v/4) + 4h + v%4
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 o = f32x4{oacc[t][4 * j], oacc[t][4 * j + 1], oacc[t][4 * j + 2],
                            oacc[t][4 * j + 3]} * inv;
      *reinterpret_cast<f32x4*>(dst + 32 * t + 8 * j + 4 * h) = o;
    }
}

template <int D, int NRG, int KS>
hipError_t launch_t(const ChunkAttnArgs& a, hipStream_t stream) {
  const int rows = a.q_len * a.G;
  const int tiles = (rows + 32 * NRG - 1) / (32 * NRG);
  const dim3 blocks(a.n_kv_heads * a.num_splits * tiles);
  const dim3 threads(NRG * KS * 64);
  if (a.pt != nullptr) return launch_kernel(prefill_attn_kernel<D, NRG, KS, true>, blocks, threads, a, stream);
  return launch_kernel(prefill_attn_kernel<D, NRG, KS, false>, blocks, threads, a, stream);
}

template <int D>
hipError_t launch_d(const ChunkAttnArgs& a, hipStream_t stream) {
  const int tile = prefill_tile_rows(a.q_len * a.G, a.n_kv_heads, a.num_splits, a.fill_wgs);
  if (tile == kPrefillTileRows) return launch_t<D, kPrefillTileRows / 32, 1>(a, stream);
  if (tile == kPrefillTileRows / 2) return launch_t<D, kPrefillTileRows / 64, 2>(a, stream);
  return launch_t<D, kPrefillTileRows / 128, 2>(a, stream);
}

}  // namespace

hipError_t launch_prefill_attn(const ChunkAttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  return launch_d<64>(a, stream);
}

}  // namespace rkv
