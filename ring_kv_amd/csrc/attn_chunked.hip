// Verify-block attention over a chunked KV store: the paged pool of 64-token chunks
// (lucebox post "Laguna XS 2.1 33B on a RTX 3090: 296 tok/s peak, 152 tok/s at 256K
// context", "Three optimizations", item 1) and the sliding-window position ring (same
// post, "3. Ring caches for the sliding-window layers").  The ring is a store of
// ring_size/64 chunk slots in which logical chunk c sits in slot c mod (ring_size/64), so
// both stores go through one kernel that differs only in the chunk -> slot rule.
//
// One workgroup = one KV head g, one range of whole chunks (a split) and one tile of 64 of the
// q_len * G (query, query-head) rows that read head g.  Its 8 waves are 4 row groups x 2 key
// halves: wave (rg, kh) owns rows 16rg .. 16rg+15 of the tile and keys 32kh .. 32kh+31 of every
// chunk, keeps its own online-softmax state, and the two halves of a row group merge their
// states through LDS at the end.  Per chunk, for every wave:
//   S^T [32 keys x 16 rows] = K [32 x D] . Q^T       2 x (D/32) MFMA 16x16x32 bf16
//   online softmax over its 32 keys per row           (f32, exp2 domain)
//   O^T [D x 16 rows]     += V^T [D x 32] . P^T       D/16 MFMA, plus one for the row sum
// Computing S transposed leaves each lane with scores of ONE row, which is exactly the
// B-operand layout of P^T for the second product: no LDS round trip for P.  Within a pair
// of 16-key tiles the key order is permuted (sigma below) so that each lane's 8 P values
// are 8 consecutive keys, which the dimension-major V chunk supplies as one 16-byte read.
//
// A ring layer can run as one launch (FUSE): the split workgroups of each (KV head, row tile)
// are placed on one XCD, store their partials, wait for each other through a counter in the
// workspace, and each merges a share of the tile's rows; otherwise a second launch merges the
// partials (attn_merge.hip), with the same bits.
//
// Memory path: K and V chunks stream from HBM with 16-byte loads (a wave reads 1 KiB contiguous
// per instruction) two chunks ahead of the compute, staged in registers and written into two
// XOR-swizzled LDS tiles that all waves read.  (The direct HBM-to-LDS loads of gfx950 were
// measured here at ~6 TB/s against ~7 TB/s for register loads of the same blocks, so the data
// takes the register path.)
#include "rkv_device.hpp"
#include "rkv_launch.hpp"

#include <type_traits>

namespace rkv {

namespace {

// S^T row m of 16-key tile tm -> key within the chunk.  Lane group q of the C layout holds
// rows 4q..4q+3 of each tile; tiles 2ks and 2ks+1 together give that lane keys
// 32ks + 8q + 0..7.
__device__ __forceinline__ int sigma(int tm, int m) {
  return 32 * (tm >> 1) + 8 * (m >> 2) + 4 * (tm & 1) + (m & 3);
}

// XOR swizzles of the 16-byte pieces inside an LDS row.  A K read of one MFMA operand touches
// 16 keys (bits 0,1,3,4 of the key vary) at one piece; a V^T read touches 16 consecutive rows
// d.  The swizzles give every group of 8 lanes 8 distinct 16-byte slots of a 128-byte bank
// line and every group of 16 lanes 16 distinct slots of a 256-byte line.
template <int D>
__device__ __forceinline__ int swz_k(int key) {
  return D == 128 ? ((key & 3) | ((key >> 1) & 12)) : ((key & 3) | ((key >> 1) & 4));
}
__device__ __forceinline__ int swz_v(int d) { return ((d >> 1) & 7) ^ ((d & 1) << 2); }

// Lazy rescaling: a row keeps its running max until a score exceeds it by more than this
// (exp2 domain), so weights stay below 2^8 and the accumulators are rescaled only rarely.
constexpr float kRescaleSlack = 8.0f;

// max over the four lanes of a row (lanes n, n+16, n+32, n+48): gfx950 row-swap permutes
__device__ __forceinline__ float row_max4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// sum over the four lanes of a row, the same value (and the same bits) on all four
__device__ __forceinline__ float row_sum4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Positions inside a workgroup are 32-bit offsets from its split's first key, clamped to
// +-2^29 (a split spans at most kMaxSplitChunks chunks, 2^28 positions), so every edge test is a
// 32-bit scalar or vector compare.
__device__ __forceinline__ int rel_pos(int64_t x, int64_t base) {
  return (int)imax64(-(int64_t(1) << 29), imin64(x - base, int64_t(1) << 29));
}

constexpr int kPtCap = 512;   // page-table entries kept in LDS (a power of two, >= 512)

template <int D>
struct Tile {
  static constexpr int kRow = D / 8;           // 16-byte pieces per K row
  static constexpr int kPieces = 64 * kRow;    // K pieces per chunk
  static constexpr int vPieces = D * 8;        // V pieces per chunk (D rows of 64 keys)
  static constexpr int elems = 2 * 64 * D;     // bf16 elements per LDS buffer
  // LDS offsets in bf16 elements
  __device__ static __forceinline__ int k_off(int key, int piece) {
    return key * D + ((piece ^ swz_k<D>(key)) << 3);
  }
  __device__ static __forceinline__ int v_off(int d, int piece) {
    return 64 * D + d * 64 + ((piece ^ swz_v(d)) << 3);
  }
};

// hardware register XCC_ID (id 20, all 32 bits): the XCD the wave runs on
constexpr int kHwRegXccId = 20 | (31 << 11);

// The counter line of a (KV head, row tile) group in the one-launch ring layer holds two words.
// Word 0 counts this launch's arrivals (bits 0..4) and sums the arrivals' XCD ids plus one
// (bits 10..17, at most 12 x 16) and their squares (bits 18..29, at most 12 x 256): equal sums of
// ids and of squared ids (S times one id and S times its square) force every id to be that one.
// The last arrival resets it to zero.  Word kGenWord is a generation that only the last arrival
// of a launch moves (by 1 if the group checked out, by 2 if not), so the others wait for it to
// move from the value they read before arriving; it needs no reset.
constexpr int kArrive = 1;
constexpr int kGenWord = 16;           // ints: the generation sits 64 bytes into the line
constexpr int kSpinLimit = 1 << 17;    // polls before a workgroup gives up (NaN rows)

// cache policy sc1 of a buffer store (gfx950): written through the XCD's L2
constexpr int kSc1 = 16;

// This workgroup's share of the merge of its (KV head g, row tile) group's partials, once every
// workgroup of the group has stored its own: local rows s, s + S, s + 2S, ... of the tile.  The
// arithmetic is merge_kernel's (the same weights, the same split groups summed in the same
// order), so both paths give the same bits.  Each pass takes RPP rows, D/4 threads per row, each
// owning four output dimensions, so a wave instruction reads whole 4*D-byte partial rows; the
// split weights of a row are computed once (one exponential per thread) and shared through
// LDS.  Loads miss the L1 (cache policy sc0); the partials, stored through the XCD's L2 and
// acknowledged before each arrival, come from that L2 or from memory.  bad: write NaN instead
// (a workgroup of the group ran on another XCD, or never arrived).
template <int D, int NT, int ROWS>
__device__ __forceinline__ void merge_share(const ChunkAttnArgs& a, int g, int row0, int s,
                                            bool bad) {
  constexpr int PR = D / 4;                       // four-element columns per row
  constexpr int RPP = NT / PR;                    // rows per pass
  constexpr int SG = merge_groups<D>();
  static_assert(NT % PR == 0 && PR >= kFuseMaxSplits && kFuseMaxSplits % 4 == 0, "merge layout");
  __shared__ __attribute__((aligned(16))) float w_sh[RPP][kFuseMaxSplits];
  const int rows = a.q_len * a.G;
  const int S = a.num_splits;
  const int tid = threadIdx.x;
  const int col = tid % PR;
  const int slot = tid / PR;
  const uint32_t prows = (uint32_t)(a.n_kv_heads * S * rows);
  const __amdgpu_buffer_rsrc_t po =
      __builtin_amdgcn_make_buffer_rsrc(a.part_o, 0, prows * D * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t pl =
      __builtin_amdgcn_make_buffer_rsrc(a.part_lse, 0, prows * 4, 0x00020000);
  const int mine = (ROWS - s + S - 1) / S;        // local rows of this workgroup
  const float nan = __builtin_nanf("");
  for (int q0 = 0; q0 < mine; q0 += RPP) {
    const int lr = s + S * (q0 + slot);           // local row of this thread
    const int r = min(row0 + lr, rows - 1);       // clamped: every load is in range
    auto prow_of = [&](int k) __attribute__((always_inline)) {
      return (uint32_t)((g * S + min(k, S - 1)) * rows + r);
    };
    float lv[kFuseMaxSplits];
    f32x4 ov[kFuseMaxSplits];
#pragma unroll
    for (int k = 0; k < kFuseMaxSplits; ++k) {
      lv[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pl, prow_of(k) * 4, 0, 1));
      ov[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            po, (prow_of(k) * D + 4 * col) * 4, 0, 1));
    }
    const float l_col = col < kFuseMaxSplits
        ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pl, prow_of(col) * 4, 0, 1))
        : 0.f;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kFuseMaxSplits; ++k)
      if (k < S) M = fmaxf(M, lv[k]);
    const float Mu = M == -INFINITY ? 0.f : M;
    if (col < kFuseMaxSplits) w_sh[slot][col] = col < S ? merge_weight(l_col, Mu) : 0.f;
    lds_barrier();
    float wv[kFuseMaxSplits];
#pragma unroll
    for (int k4 = 0; k4 < kFuseMaxSplits / 4; ++k4) {
      const f32x4 w4 = *reinterpret_cast<const f32x4*>(&w_sh[slot][4 * k4]);
      wv[4 * k4] = w4[0]; wv[4 * k4 + 1] = w4[1]; wv[4 * k4 + 2] = w4[2]; wv[4 * k4 + 3] = w4[3];
    }
    if (q0 + slot < mine && row0 + lr < rows) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      float Lt = 0.f;
#pragma unroll
      for (int sg = 0; sg < SG; ++sg) {
        f32x4 acc_g = f32x4{0.f, 0.f, 0.f, 0.f};
        float L_g = 0.f;
        // splits k >= S weigh exactly 0 here: adding o * 0 = +-0 to a sum that is never -0 (it
        // starts at +0, and a sum that cancels to zero is +0) leaves its bits as merge_kernel's,
        // which skips them; a NaN partial still makes the row NaN
#pragma unroll
        for (int k = sg; k < kFuseMaxSplits; k += SG) merge_add(acc_g, L_g, ov[k], wv[k]);
        Lt += L_g;
        if (sg == 0) acc = acc_g;
        else acc += acc_g;
      }
      const int qi = r / a.G;
      const int h = g * a.G + r % a.G;
      *reinterpret_cast<f32x4*>(a.out + ((int64_t)qi * a.n_q_heads + h) * D + 4 * col) =
          bad ? f32x4{nan, nan, nan, nan} : merge_out(acc, Lt);
      if (a.lse != nullptr && col == 0)
        a.lse[(int64_t)qi * a.n_q_heads + h] = bad ? nan : merge_lse(M, Lt);
    }
    lds_barrier();                                // w_sh is rewritten by the next pass
  }
}

// Template parameters:
//   NRG    row groups: wave (rg, kh) owns rows 16*rg .. 16*rg+15 of the KV head's rows
//   KS     key halves: with KS = 2 each chunk's 64 keys are split between two waves per row
//          group (keys 0..31 and 32..63); each keeps its own online-softmax state and the two
//          states merge through LDS at the end.  Two waves per SIMD, each with half the
//          dependent work per chunk.
//   PAGED  slots come from the page table; otherwise the store is a ring (slot = c mod n_slots)
//   FUSE   the one-launch layer: the workgroups of each (KV head, row tile) merge the tile's
//          partials once all are stored (see merge_share above); the grid is one-dimensional
//   APPEND the block's own rows come from k_new / v_new and are written into the store by this
//          launch (a separate instantiation, so that the other launches carry none of its code)
template <int D, int NRG, int KS, bool PAGED, bool FUSE, bool APPEND>
__global__ __launch_bounds__(NRG * KS * 64)
void chunk_attn_kernel(ChunkAttnArgs a) {
  using T = Tile<D>;
  constexpr int NW = NRG * KS;
  constexpr int NT = NW * 64;
  // Chunks in flight = register stages NST; chunk loc goes through stage loc % NST and LDS
  // tile loc % NLDS.  Two tiles suffice: the barrier of step loc - 1 follows every wave's
  // compute of chunk loc - 2, the last reader of the tile that step loc overwrites.
  constexpr int NST = 2;
  constexpr int NLDS = 2;
  static_assert(NST % NLDS == 0 && NST >= 2 && NST <= 4, "stage / tile counts");
  constexpr int LPC = (T::kPieces + T::vPieces) / NT;   // 16-byte loads per chunk per thread
  static_assert((T::kPieces + T::vPieces) % NT == 0, "pieces must divide evenly");
  static_assert(T::kPieces % NT == 0, "a load index is all K or all V for every thread");
  constexpr int PF = NST;                                // chunks in flight ahead of compute
  constexpr int KK = D / 32;
  constexpr int TMD = D / 16;
  constexpr int NKS = KS == 2 ? 1 : 2;                   // 32-key halves per wave per chunk

  __shared__ __attribute__((aligned(16))) uint16_t lds[NLDS][T::elems];
  __shared__ int pt_lds[kPtCap];
  __shared__ int wave_flag[NW];   // per wave: a table entry of the split is out of range
  __shared__ int merge_flag;      // FUSE: 1 the group's partials are all stored, 2 write NaN

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = w % NRG;
  const int kh = w / NRG;
  const int ln = lane & 15;
  const int lq = lane >> 4;

  int g, s, tile, grp = 0;
  uint32_t gen0 = 0;               // FUSE: the group's generation before this launch's arrivals
  if constexpr (FUSE) {
    // The S workgroups of group grp = (KV head, row tile) are blocks x, x + 8, x + 16, ... of
    // one residue x mod 8: the dispatcher deals blocks round-robin over the 8 XCDs, so a group
    // runs on one XCD and shares its L2.
    const int per_xcd = gridDim.x / kXcds;
    const int j = blockIdx.x / kXcds;
    grp = (blockIdx.x % kXcds) * (per_xcd / a.num_splits) + j / a.num_splits;
    s = j % a.num_splits;
    g = grp % a.n_kv_heads;
    tile = grp / a.n_kv_heads;
    // read now, long before this workgroup arrives: only the group's last arrival moves it
    if (tid == 0)
      gen0 = (uint32_t)__hip_atomic_fetch_add(a.tickets + grp * (kTicketStride / 4) + kGenWord, 0,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    const int b = xcd_block(blockIdx.x, gridDim.x);
    g = b % a.n_kv_heads;
    s = b / a.n_kv_heads;
    tile = blockIdx.y;
  }
  const int G = a.G;
  const int rows = a.q_len * G;

  // Positions of the block: from the arguments, or derived from the device-resident position
  // of its first row (one captured step replayed as the context grows).  A pool split's first
  // chunk does not depend on it (pool keys start at position 0), so the first table reads need
  // not wait for it.
  int64_t p0 = a.p0, valid_lo = a.valid_lo, valid_hi = a.valid_hi;
  int64_t c_first = PAGED ? 0 : a.c_first, n_chunks = a.n_chunks;
  bool pos_bad = false;
  if (a.d_pos != nullptr) {
    const int64_t P = *a.d_pos;
    pos_bad = P < 0 || P > a.pos_cap;
    p0 = pos_bad ? 0 : P;
    const int64_t end = p0 + a.q_len;
    valid_hi = end;
    if (PAGED) {
      valid_lo = 0;
      n_chunks = (end + kChunk - 1) / kChunk;
    } else {
      const int64_t lo = a.window > 0 ? imax64(0, p0 - a.window + 1) : 0;
      c_first = lo / kChunk;
      n_chunks = (end - 1) / kChunk - c_first + 1;
      valid_lo = imax64(0, end - a.ring_size);
    }
  }

  const int64_t c_lo = c_first + (int64_t)s * a.cps;
  const int64_t c_end = c_first + n_chunks;
  const int nloc = (int)imax64(0, imin64((int64_t)a.cps, c_end - c_lo));

  // ---- the block's own rows, appended by this launch ------------------------------------------
  // A workgroup whose range of several chunks holds positions of the block writes those rows
  // into their slots before it reads any chunk (K rows as 16-byte pieces, V into its
  // dimension-major rows), and waits for the stores: its chunk loads then see them.  Several
  // workgroups (the row tiles of a range) write the same bytes.  (A one-chunk range lays the
  // rows over its tile in LDS instead, below.)  A device position out of range writes nothing;
  // a pool chunk whose table entry lies outside the pool is skipped (the attention masks that
  // chunk).
  if (APPEND && !pos_bad && nloc > 1) {
    const int64_t b_lo = imax64(p0, c_lo * kChunk);
    const int64_t b_hi = imin64(p0 + a.q_len, (c_lo + nloc) * kChunk);
    if (b_lo < b_hi) {
      constexpr int PC = D / 8;                      // 16-byte pieces per row
      const int nrow = (int)(b_hi - b_lo);
      for (int u = threadIdx.x; u < nrow * PC; u += NRG * KS * 64) {
        const int j = u / PC, pc = u % PC;
        const int64_t pos = b_lo + j;
        const int64_t c = pos / kChunk;
        const int64_t slot = PAGED ? (int64_t)a.pt[c] : c % a.n_slots;
        if (slot < 0 || slot >= a.n_slots) continue;
        const int off = (int)(pos % kChunk);
        const int64_t src = ((pos - p0) * a.n_kv_heads + g) * D + pc * 8;
        const int64_t blk = slot * a.n_kv_heads + g;
        const u32x4 kv = *reinterpret_cast<const u32x4*>(a.k_new + src);
        const u32x4 vv = *reinterpret_cast<const u32x4*>(a.v_new + src);
        *reinterpret_cast<u32x4*>(a.k_w + (blk * kChunk + off) * D + pc * 8) = kv;
        uint16_t* vd = a.v_w + (blk * D + pc * 8) * kChunk + off;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vd[(2 * e) * kChunk] = (uint16_t)(vv[e] & 0xffffu);
          vd[(2 * e + 1) * kChunk] = (uint16_t)(vv[e] >> 16);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // ---- this lane's query row (row tile y holds rows 16*NRG*y ..) ---------------------------
  const int row0 = tile * (NRG * 16);
  const int r = row0 + rg * 16 + ln;
  const bool row_ok = r < rows;
  const int qi = row_ok ? r / G : 0;
  const int hq = g * G + (row_ok ? r % G : 0);
  const bool wave_active = row0 + rg * 16 < rows;
  // key position bounds, relative to this split's first key c_lo * 64
  const int64_t pbase = c_lo * 64;
  const int64_t p_i64 = p0 + qi;
  const int p_i = rel_pos(p_i64, pbase);                             // this row's query
  const int lo_i = rel_pos(a.window > 0 ? imax64(0, p_i64 - a.window + 1) : 0, pbase);
  const int p_first = rel_pos(p0, pbase);                            // first query of the block
  const int64_t p_last = p0 + a.q_len - 1;
  const int lo_last = rel_pos(a.window > 0 ? imax64(0, p_last - a.window + 1) : 0, pbase);
  const int vlo = rel_pos(valid_lo, pbase);                          // stored keys [vlo, vhi)
  const int vhi = rel_pos(valid_hi, pbase);

  // Q^T operand of S^T = K Q^T: lane (ln, lq) holds row ln's dims kk*32 + 8*lq .. +7
  bf16x8 qop[KK];
  auto load_q = [&]() __attribute__((always_inline)) {
    const uint16_t* qrow = a.q + ((int64_t)qi * a.n_q_heads + hq) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      // qi, hq are clamped to row 0 for rows past the end: load, then zero
      u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + kk * 32 + lq * 8);
      if (!row_ok) raw = u32x4{0u, 0u, 0u, 0u};
      qop[kk] = __builtin_bit_cast(bf16x8, raw);
    }
  };

  constexpr bool paged = PAGED;
  // ring: slot = logical chunk mod n_slots; a ring span covers at most n_slots + 1 chunks
  const int ring_base = paged ? 0 : (int)(c_lo % a.n_slots);
  auto slot_of = [&](int loc) __attribute__((always_inline)) -> int {
    if (!paged) {
      int t = ring_base + loc;
      t -= t >= a.n_slots ? a.n_slots : 0;
      t -= t >= a.n_slots ? a.n_slots : 0;
      return t;
    }
    return __builtin_amdgcn_readfirstlane(pt_lds[loc & (kPtCap - 1)]);
  };
  auto maybe_refresh_table = [&](int loc, auto refresh_tag) __attribute__((always_inline)) {
    // at loc = 256k + 128 (k >= 1) load local chunks [256(k+1), 256(k+2)) into half (k+1)&1,
    // which last held chunks [256(k-1), 256k), all issued by now
    if constexpr (!decltype(refresh_tag)::value) return;
    if (!paged || nloc <= kPtCap || (loc & 255) != 128 || loc < 256) return;
    const int base = ((loc >> 8) + 1) << 8;
    if (base >= nloc) return;
    for (int e = tid; e < 256; e += NT)
      if (base + e < nloc) pt_lds[(base + e) & (kPtCap - 1)] = a.pt[c_lo + base + e];
  };

  // Register stages: chunk loc is loaded into stage loc % NST (piece P = u*NT + tid of the chunk,
  // so each wave instruction reads 1 KiB of contiguous HBM) and written to LDS tile loc % NLDS
  // at its swizzled place.  A chunk past the split, or with an out-of-range slot, loads one line of
  // slot 0 instead (cached, never computed), so every iteration has the same loads in flight and
  // the compiler's wait counts stay exact.
  u32x4 stg0[LPC], stg1[LPC], stg2[LPC], stg3[LPC];
  int sl0 = -1, sl1 = -1, sl2 = -1, sl3 = -1;   // slot of each stage's chunk (-1: none), uniform
  auto stage = [&](auto st_tag) __attribute__((always_inline)) -> u32x4* {
    constexpr int S = decltype(st_tag)::value;
    if constexpr (S == 0) return stg0;
    else if constexpr (S == 1) return stg1;
    else if constexpr (S == 2) return stg2;
    else return stg3;
  };
  auto stage_slot = [&](auto st_tag) __attribute__((always_inline)) -> int& {
    constexpr int S = decltype(st_tag)::value;
    if constexpr (S == 0) return sl0;
    else if constexpr (S == 1) return sl1;
    else if constexpr (S == 2) return sl2;
    else return sl3;
  };
  // Branch-free on purpose: the slot, the base and a lane-offset mask are uniform selects, so
  // every step issues the same loads and the wait counts before each commit stay exact.
  // cand: the chunk's slot as the table or ring gives it (garbage past the split: masked)
  auto issue = [&](auto st_tag, int loc, int cand) __attribute__((always_inline)) {
    u32x4* st = stage(st_tag);
    const bool ok = loc < nloc && (unsigned)cand < (unsigned)a.n_slots;
    const int slot = ok ? cand : 0;
    stage_slot(st_tag) = ok ? cand : -1;
    const uint32_t keep = ok ? 0xffffffffu : 0u;        // 0: every lane reads piece 0
    const int64_t blk = (int64_t)slot * a.n_kv_heads + g;
    const uint16_t* kb = a.k + blk * (64 * D);
    const uint16_t* vb = a.v + blk * (64 * D);
#pragma unroll
    for (int u = 0; u < LPC; ++u) {
      const int P = u * NT + tid;
      const uint16_t* src = (u * NT < T::kPieces)
                                ? kb + (((uint32_t)P * 8u) & keep)
                                : vb + (((uint32_t)(P - T::kPieces) * 8u) & keep);
      st[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
    }
  };
  auto commit = [&](auto st_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(st_tag)::value;
    const u32x4* st = stage(st_tag);
    uint16_t* buf = &lds[S % NLDS][0];
#pragma unroll
    for (int u = 0; u < LPC; ++u) {
      const int P = u * NT + tid;
      int off;
      if (u * NT < T::kPieces) {
        const int key = P / T::kRow, pc = P % T::kRow;
        off = T::k_off(key, pc);
      } else {
        const int vp = P - T::kPieces;
        off = T::v_off(vp >> 3, vp & 7);
      }
      *reinterpret_cast<u32x4*>(buf + off) = st[u];
    }
  };

  // ---- running softmax state ---------------------------------------------------------
  // m_run: exp2-domain reference max of this lane's row over the wave's keys.  oacc holds
  // sum_j p_j V_j^T and lacc the row sum sum_j p_j (computed by the matrix core against a
  // column of ones, so it uses exactly the bf16 weights the PV product uses: the output's
  // normaliser).  lf is this lane's share of the same sum over the f32 weights, for the lse:
  // a row dominated by one key would otherwise carry that weight's bf16 rounding (up to 2^-8)
  // into its lse.
  float m_run = -INFINITY;
  float lf = 0.f;
  f32x4 oacc[TMD];
  f32x4 lacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < TMD; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // A operand of the ones column: row 0 of an extra 16-row tile of V^T is all ones
  const bf16x8 ones_col = __builtin_bit_cast(
      bf16x8, ln == 0 ? u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u}
                      : u32x4{0u, 0u, 0u, 0u});
  const float csc = a.scale_log2;

  // EDGE: some key of the chunk may be invisible to some row (causal tail, window start), lie
  // outside the stored range (partial) or come from no slot (ok false: the stage holds filler);
  // interior chunks run without any masking code.
  auto compute_body = [&](const uint16_t* buf, int cbase, bool partial, bool ok, auto edge_tag) __attribute__((always_inline)) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    f32x4 sacc[2 * NKS];
#pragma unroll
    for (int j = 0; j < 2 * NKS; ++j) sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8 ka[2 * NKS];
#pragma unroll
      for (int j = 0; j < 2 * NKS; ++j) {
        const int tm = 2 * (KS == 2 ? kh : (j >> 1)) + (j & 1);
        ka[j] = *reinterpret_cast<const bf16x8*>(buf + T::k_off(sigma(tm, ln), 4 * kk + lq));
      }
#pragma unroll
      for (int j = 0; j < 2 * NKS; ++j) sacc[j] = mfma_16x16x32(ka[j], qop[kk], sacc[j]);
    }
    // key index within the chunk of score (j, i): 32*ks + 8*lq + 4*(j&1) + i
    float mx = -INFINITY;
    if constexpr (EDGE) {
      // visible keys of this row: [vis_lo, vis_hi] relative to the chunk
      const int vis_lo = max(-1, min(max(lo_i, vlo) - cbase, 64));
      const int vis_hi = (row_ok && ok) ? max(-1, min(min(p_i, vhi - 1) - cbase, 64)) : -1;
#pragma unroll
      for (int j = 0; j < 2 * NKS; ++j) {
        const int ks = KS == 2 ? kh : (j >> 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kidx = 32 * ks + 8 * lq + 4 * (j & 1) + i;
          // selection, not arithmetic: a key outside the stored range may hold anything
          if (kidx < vis_lo || kidx > vis_hi) sacc[j][i] = -INFINITY;
          mx = fmaxf(mx, sacc[j][i]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2 * NKS; ++j)
        mx = fmaxf(mx, fmaxf(fmaxf(sacc[j][0], sacc[j][1]), fmaxf(sacc[j][2], sacc[j][3])));
    }
    const float t_max = row_max4(mx) * csc;          // scale > 0: max commutes with it
    // rescale only when some row's max passed its reference by more than the slack
    const bool grow = t_max > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? t_max : m_run;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;   // -inf -> 0
#pragma unroll
      for (int t = 0; t < TMD; ++t) oacc[t] *= alpha;
      lacc *= alpha;
      lf *= alpha;
      m_run = m_new;
    }
    // a row with no visible key yet keeps m_run = -inf; its weights must come out 0, not NaN
    const float m_use = (EDGE && m_run == -INFINITY) ? 0.f : m_run;
    uint32_t pw[NKS][4];   // P^T operand words per 32-key half
#pragma unroll
    for (int h = 0; h < NKS; ++h) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int j = 2 * h + hh;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[j][0], csc, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[j][1], csc, -m_use));
        const float p2 = __builtin_amdgcn_exp2f(fmaf(sacc[j][2], csc, -m_use));
        const float p3 = __builtin_amdgcn_exp2f(fmaf(sacc[j][3], csc, -m_use));
        pw[h][2 * hh] = pack_bf16x2(p0, p1);
        pw[h][2 * hh + 1] = pack_bf16x2(p2, p3);
        lf += (p0 + p1) + (p2 + p3);
      }
    }
#pragma unroll
    for (int h = 0; h < NKS; ++h) {
      const int ks = KS == 2 ? kh : h;
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pw[h][0], pw[h][1], pw[h][2], pw[h][3]});
      uint32_t vmask[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
      if constexpr (EDGE) {
        // keys outside the stored range or without a slot: zero their V so that
        // 0 * (anything) stays 0
        if (partial || !ok) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int jj = cbase + 32 * ks + 8 * lq + e;
            if (!ok || jj < vlo || jj >= vhi) vmask[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          }
        }
      }
#pragma unroll
      for (int t = 0; t < TMD; ++t) {
        u32x4 raw = *reinterpret_cast<const u32x4*>(buf + T::v_off(16 * t + ln, 4 * ks + lq));
        if constexpr (EDGE) {
          raw[0] &= vmask[0]; raw[1] &= vmask[1]; raw[2] &= vmask[2]; raw[3] &= vmask[3];
        }
        oacc[t] = mfma_16x16x32(__builtin_bit_cast(bf16x8, raw), pb, oacc[t]);
      }
      lacc = mfma_16x16x32(ones_col, pb, lacc);
    }
  };

  // Every wave computes every chunk it is given, even a wave whose rows are all past the end
  // (its Q is zero and nothing of it is written): a skip would be a control-flow join at which
  // the compiler copies all accumulators.
  auto compute = [&](const uint16_t* buf, int loc, int slot, auto edge_tag) __attribute__((always_inline)) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const int cbase = loc * 64;
    if constexpr (EDGE) {
      const bool partial = cbase < vlo || cbase + 64 > vhi;
      compute_body(buf, cbase, partial, (unsigned)slot < (unsigned)a.n_slots, std::true_type{});
    } else {
      compute_body(buf, cbase, false, true, std::false_type{});
    }
  };

  // A one-chunk split takes the masking path when its chunk meets the window start, the causal
  // tail or an end of the stored range.
  const bool span_edge = nloc > 0 && ((nloc - 1) * 64 + 63 > p_first || lo_last > 0 ||
                                      vlo > 0 || nloc * 64 > vhi);

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  if (nloc <= 1) {
    // ---- one chunk (the ring's default split): its loads and Q's go out together -------
    const int cand = paged ? (nloc == 1 ? __builtin_amdgcn_readfirstlane(a.pt[c_lo]) : -1)
                           : ring_base;
    issue(I0{}, 0, cand);
    load_q();
    // Block rows in this chunk (appended by this launch): requested with the chunk and Q, laid
    // over the chunk's tile once it is in LDS, and written into the slot by the first row tile.
    const int64_t pb_lo = imax64(p0, c_lo * kChunk);
    const int pnrow = (int)imax64(0, imin64(p0 + a.q_len, (c_lo + 1) * kChunk) - pb_lo);
    const bool patch = APPEND && !pos_bad && nloc == 1 && pnrow > 0;
    constexpr int PCS = D / 8;                // 16-byte pieces per row
    constexpr int MAXU = 2;                   // pieces per thread kept in registers
    u32x4 pk[MAXU], pv[MAXU];
    auto new_piece = [&](int e) __attribute__((always_inline)) {
      return ((pb_lo - p0 + e / PCS) * a.n_kv_heads + g) * D + (e % PCS) * 8;
    };
    if (patch) {
#pragma unroll
      for (int u = 0; u < MAXU; ++u) {
        const int e = tid + u * NT;
        if (e < pnrow * PCS) {
          pk[u] = *reinterpret_cast<const u32x4*>(a.k_new + new_piece(e));
          pv[u] = *reinterpret_cast<const u32x4*>(a.v_new + new_piece(e));
        }
      }
    }
    commit(I0{});
    lds_barrier();
    if (patch) {
      const bool write = tile == 0 && (unsigned)cand < (unsigned)a.n_slots;
      const int64_t blk = (int64_t)cand * a.n_kv_heads + g;
      const int key0 = (int)(pb_lo - c_lo * kChunk);
      auto lay = [&](int e, const u32x4& kv, const u32x4& vv) __attribute__((always_inline)) {
        const int key = key0 + e / PCS, pc = e % PCS;
        uint16_t* buf = &lds[0][0];
        *reinterpret_cast<u32x4*>(buf + T::k_off(key, pc)) = kv;
#pragma unroll
        for (int h2 = 0; h2 < 8; ++h2) {
          const uint32_t w2 = vv[h2 >> 1];
          buf[T::v_off(pc * 8 + h2, key >> 3) + (key & 7)] =
              (uint16_t)((h2 & 1) ? (w2 >> 16) : (w2 & 0xffffu));
        }
        if (write) {
          *reinterpret_cast<u32x4*>(a.k_w + (blk * kChunk + key) * D + pc * 8) = kv;
          uint16_t* vd = a.v_w + (blk * D + pc * 8) * kChunk + key;
#pragma unroll
          for (int h2 = 0; h2 < 8; ++h2) {
            const uint32_t w2 = vv[h2 >> 1];
            vd[h2 * kChunk] = (uint16_t)((h2 & 1) ? (w2 >> 16) : (w2 & 0xffffu));
          }
        }
      };
#pragma unroll
      for (int u = 0; u < MAXU; ++u) {
        const int e = tid + u * NT;
        if (e < pnrow * PCS) lay(e, pk[u], pv[u]);
      }
      for (int e = tid + MAXU * NT; e < pnrow * PCS; e += NT)   // blocks of more rows
        lay(e, *reinterpret_cast<const u32x4*>(a.k_new + new_piece(e)),
            *reinterpret_cast<const u32x4*>(a.v_new + new_piece(e)));
      lds_barrier();
    }
    if (nloc == 1) {
      if (span_edge || (unsigned)cand >= (unsigned)a.n_slots)
        compute(&lds[0][0], 0, cand, std::true_type{});
      else
        compute(&lds[0][0], 0, cand, std::false_type{});
    }
  } else {
    // The slots of the first NST chunks are read before anything else, and those chunks'
    // loads go out as soon as these reads return, while the table slice and Q are still on
    // their way (vector loads complete in order, so waiting for the first reads does not wait
    // for the later ones).  A paged split would otherwise spend one round trip on its table
    // before its first chunk load.
    int first[NST];
#pragma unroll
    for (int j = 0; j < NST; ++j)
      first[j] = paged ? a.pt[c_lo + min(j, nloc - 1)] : slot_of(j);
    // ---- page-table slice in LDS: entry for local chunk loc at pt_lds[loc % kPtCap] ---
    // kPtCap / NT entries per thread for the first kPtCap chunks; splits longer than that
    // refresh one half of the slice at a time, 128 chunks before it is needed (and always take
    // the masking path, as their later entries are not checked here).
    constexpr int TPT = kPtCap / NT;
    static_assert(kPtCap % NT == 0, "whole table entries per thread");
    int tval[TPT];
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int e = tid + j * NT;
      tval[j] = (paged && e < nloc) ? a.pt[c_lo + e] : 0;
    }
    load_q();

    // ---- pipeline: NST chunks in flight in registers while one is computed -------------
    // Step loc: write chunk loc from its register stage into LDS tile loc % NLDS, refill that
    // stage with chunk loc + NST, barrier, compute chunk loc.  The scheduler may not reorder
    // the first issues: stage 0 must hold the oldest chunk loads in flight.
    __builtin_amdgcn_sched_barrier(0);
    issue(I0{}, 0, __builtin_amdgcn_readfirstlane(first[0]));
    __builtin_amdgcn_sched_barrier(0);
    issue(I1{}, 1, __builtin_amdgcn_readfirstlane(first[1]));
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NST > 2) {
      issue(I2{}, 2, __builtin_amdgcn_readfirstlane(first[2]));
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NST > 3) {
      issue(I3{}, 3, __builtin_amdgcn_readfirstlane(first[3]));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (paged) {
      bool bad = false;
#pragma unroll
      for (int j = 0; j < TPT; ++j) {
        const int e = tid + j * NT;
        if (e < nloc) {
          pt_lds[e] = tval[j];
          bad |= (unsigned)tval[j] >= (unsigned)a.n_slots;
        }
      }
      if (lane == 0) wave_flag[w] = __builtin_amdgcn_ballot_w64(bad) != 0;
    }
    // Q has arrived before the loop: left pending, the wait-count analysis would merge its
    // loads into the chunk loop and wait on them at every use.
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(qop[kk]));
    lds_barrier();
    bool table_bad = false;     // some table entry of the split is out of range
    if (paged) {
#pragma unroll
      for (int i = 0; i < NW; ++i) table_bad |= wave_flag[i] != 0;
    }

    auto step = [&](auto st_tag, int loc, auto edge_tag, auto refresh_tag, bool refill) __attribute__((always_inline)) {
      constexpr int S = decltype(st_tag)::value;
      const int slot = stage_slot(st_tag);      // chunk loc's, before the stage is refilled
      commit(st_tag);
      maybe_refresh_table(loc + PF, refresh_tag);
      if (refill) issue(st_tag, loc + PF, slot_of(loc + PF));
      lds_barrier();
      compute(&lds[S % NLDS][0], loc, slot, edge_tag);
    };
    // The loop body is NST unconditional steps (one per stage), so the same loads are in
    // flight at every commit and the wait counts stay exact; the last NST - 1 chunks at most
    // run after it.
    // Loops of NST steps from loc (a multiple of NST) up to limit (a multiple of NST), every
    // step refilling its stage with a chunk of the split; then the last NST .. 2*NST - 1
    // chunks, which refill only while chunks remain (no load left in flight at the end).
    auto loop = [&](int& loc, int limit, auto edge_tag, auto refresh_tag) __attribute__((always_inline)) {
      for (; loc < limit; loc += NST) {
        step(I0{}, loc, edge_tag, refresh_tag, true);
        step(I1{}, loc + 1, edge_tag, refresh_tag, true);
        if constexpr (NST > 2) step(I2{}, loc + 2, edge_tag, refresh_tag, true);
        if constexpr (NST > 3) step(I3{}, loc + 3, edge_tag, refresh_tag, true);
      }
    };
    auto tail = [&](int loc, auto refresh_tag) __attribute__((always_inline)) {
      auto one = [&](auto st_tag, int j) __attribute__((always_inline)) {
        if (loc + j < nloc)
          step(st_tag, loc + j, std::true_type{}, refresh_tag, loc + j + NST < nloc);
      };
      one(I0{}, 0);
      one(I1{}, 1);
      if constexpr (NST == 2) {
        one(I0{}, 2);
      } else if constexpr (NST == 3) {
        one(I2{}, 2); one(I0{}, 3); one(I1{}, 4);
      } else {
        one(I2{}, 2); one(I3{}, 3); one(I0{}, 4); one(I1{}, 5); one(I2{}, 6);
      }
    };
    const int full = nloc >= NST ? (nloc - NST) / NST * NST : 0;
    int loc = 0;
    if (paged && nloc > kPtCap) {
      // a split longer than the table slice refreshes it from inside the loop; that load's
      // wait would lower the wait counts of every step, so these splits have a loop of their own
      loop(loc, full, std::true_type{}, std::true_type{});
      tail(loc, std::true_type{});
    } else {
      // interior chunks [a, b): at or after every row's window start and the stored range's
      // start, ending at or before the first query and the stored range's end; the chunks
      // before and after take the masking path, on boundaries that are multiples of NST
      int a = 0, b = 0;
      if (!table_bad) {
        const int lead = (max(max(lo_last, vlo), 0) + 63) / 64;
        const int end = max(min(p_first + 1, vhi), 0) / 64;
        a = min((lead + NST - 1) / NST * NST, full);
        b = max(a, min(end / NST * NST, full));
      }
      loop(loc, a, std::true_type{}, std::false_type{});
      loop(loc, b, std::false_type{}, std::false_type{});
      loop(loc, full, std::true_type{}, std::false_type{});
      tail(loc, std::false_type{});
    }
  }

  // ---- epilogue ------------------------------------------------------------------------
  // row sum: component 0 of lacc in lane ln (lane group 0); every lane of the row needs it
  float l = __shfl(lacc[0], ln, kWave);
  float lfr = row_sum4(lf);
  if constexpr (KS == 2) {
    // The two key halves of a row group exchange their states through LDS, and each combines
    // half of the row's dimensions (wave kh keeps the 16-byte columns t of O in
    // [kh * TMD/2, (kh + 1) * TMD/2) and hands the other half to its partner); both compute
    // the row's combined weights from the same values, so they agree bit for bit.  Every chunk
    // load has landed.
    constexpr int TH = TMD / 2;
    float* xo = reinterpret_cast<float*>(&lds[0][0]);          // [NRG][16][D]
    float* xm = xo + NRG * 16 * D;                               // [2][NRG][16]
    float* xl = xm + 2 * NRG * 16;
    float* xf = xl + 2 * NRG * 16;
    static_assert((NRG * 16 * D + 6 * NRG * 16) * 4 <= NLDS * T::elems * 2, "exchange fits");
    // row (rg, ln), 16-byte column 4t + lq of D/4, XOR-swizzled by the row so that the 16
    // lanes of one access group (16 rows, same column) land in 16 different bank groups
    auto xo_off = [&](int t) __attribute__((always_inline)) {
      return (rg * 16 + ln) * D + (((4 * t + lq) ^ ln) << 2);
    };
    const int r16 = rg * 16 + ln;
    lds_barrier();
    if (wave_active) {
      if (kh == 0) {
#pragma unroll
        for (int t = TH; t < TMD; ++t) *reinterpret_cast<f32x4*>(&xo[xo_off(t)]) = oacc[t];
      } else {
#pragma unroll
        for (int t = 0; t < TH; ++t) *reinterpret_cast<f32x4*>(&xo[xo_off(t)]) = oacc[t];
      }
      if (lq == 0) {
        xm[kh * NRG * 16 + r16] = m_run;
        xl[kh * NRG * 16 + r16] = l;
        xf[kh * NRG * 16 + r16] = lfr;
      }
    }
    lds_barrier();
    if (wave_active) {
      const float m0 = xm[r16], m1 = xm[NRG * 16 + r16];
      const float M = fmaxf(m0, m1);
      const float Mu = M == -INFINITY ? 0.f : M;
      const float a0 = __builtin_amdgcn_exp2f(m0 - Mu);
      const float a1 = __builtin_amdgcn_exp2f(m1 - Mu);
      l = a0 * xl[r16] + a1 * xl[NRG * 16 + r16];
      lfr = a0 * xf[r16] + a1 * xf[NRG * 16 + r16];
      if (kh == 0) {
#pragma unroll
        for (int t = 0; t < TH; ++t) {
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(&xo[xo_off(t)]);
          oacc[t] = oacc[t] * a0 + o1 * a1;
        }
      } else {
#pragma unroll
        for (int t = TH; t < TMD; ++t) {
          const f32x4 o0 = *reinterpret_cast<const f32x4*>(&xo[xo_off(t)]);
          oacc[t] = o0 * a0 + oacc[t] * a1;
        }
      }
      m_run = M;
    }
  }
  auto store_rows = [&]() __attribute__((always_inline)) {
    // a device position out of range: every output of the call is NaN
    const float inv = pos_bad ? __builtin_nanf("") : (l > 0.f ? 1.f / l : 0.f);
    const float lse_nat = pos_bad ? __builtin_nanf("")
                                  : (lfr > 0.f ? (m_run + log2f(lfr)) * kLn2 : -INFINITY);
    // with two key halves each stores its half of the columns, the first the lse
    const int t_lo = KS == 2 ? kh * (TMD / 2) : 0;
    const bool lse_lane = lq == 0 && (KS == 1 || kh == 0);
    if (a.part_o == nullptr) {
      float* dst = a.out + ((int64_t)qi * a.n_q_heads + hq) * D;
      if (a.lse != nullptr && lse_lane) a.lse[(int64_t)qi * a.n_q_heads + hq] = lse_nat;
      auto put = [&](int t) __attribute__((always_inline)) {
        *reinterpret_cast<f32x4*>(dst + 16 * t + 4 * lq) = oacc[t] * inv;
      };
      if (KS == 1) {
#pragma unroll
        for (int t = 0; t < TMD; ++t) put(t);
      } else if (t_lo == 0) {
#pragma unroll
        for (int t = 0; t < TMD / 2; ++t) put(t);
      } else {
#pragma unroll
        for (int t = TMD / 2; t < TMD; ++t) put(t);
      }
      return;
    }
    // Partials: written through the XCD's L2 (cache policy sc1), which the kernel's end then
    // need not write back (measured: a launch storing 8 MiB ends ~0.6 us sooner; the 40-layer
    // step, whose window layers store theirs for the merge inside the launch, ran ~5 us
    // faster).  Buffer bases are this (KV head, split)'s block of rows.
    const int64_t blk = ((int64_t)g * a.num_splits + s) * rows;
    const __amdgpu_buffer_rsrc_t po =
        __builtin_amdgcn_make_buffer_rsrc(a.part_o + blk * D, 0, rows * D * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t pl =
        __builtin_amdgcn_make_buffer_rsrc(a.part_lse + blk, 0, rows * 4, 0x00020000);
    if (lse_lane)
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse_nat), pl, r * 4, 0,
                                            kSc1);
    auto put = [&](int t) __attribute__((always_inline)) {
      const f32x4 o = oacc[t] * inv;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), po,
                                             (r * D + 16 * t + 4 * lq) * 4, 0, kSc1);
    };
    if (KS == 1) {
#pragma unroll
      for (int t = 0; t < TMD; ++t) put(t);
    } else if (t_lo == 0) {
#pragma unroll
      for (int t = 0; t < TMD / 2; ++t) put(t);
    } else {
#pragma unroll
      for (int t = TMD / 2; t < TMD; ++t) put(t);
    }
  };
  if constexpr (!FUSE) {
    if (!wave_active || !row_ok) return;
    store_rows();
  } else {
    if (wave_active && row_ok) store_rows();
    // ---- the group merges its partials once all of them are stored ---------------------------
    // A workgroup's partial stores are acknowledged once written through the XCD's L2; its
    // arrival follows every thread's acknowledgement.  The last of the group's S arrivals checks
    // the group and moves the generation; the others wait for it to move (a bounded poll) and
    // then every workgroup merges its share of the tile's rows.  The group's workgroups are all
    // resident at once (the launch is used only when its grid fits one workgroup per compute
    // unit), so the wait ends when the slowest of them arrives.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int* const ticket = a.tickets + grp * (kTicketStride / 4);
    int* const gen = ticket + kGenWord;
    const int S = a.num_splits;
    if (tid == 0) {
      // the XCD id plus one, so that no id sums to zero (a counter that was not zeroed cannot
      // pass for a complete group)
      const int x = (int)((uint32_t)__builtin_amdgcn_s_getreg(kHwRegXccId) & 15u) + 1;
      int arrive = kArrive + (x << 10) + ((x * x) << 18);
      // the arrival depends on the generation read at the start, so it is issued only once that
      // read has returned: every workgroup reads the generation before the last arrival moves it
      asm volatile("" : "+v"(arrive) : "v"(gen0));
      const int v = __hip_atomic_fetch_add(ticket, arrive, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) + arrive;
      int flag;
      if ((v & 31) == S) {
        const bool all_here = ((v >> 10) & 255) == S * x && ((v >> 18) & 4095) == S * x * x;
        __hip_atomic_store(gen, (int)(gen0 + (all_here ? 1u : 2u)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        flag = all_here ? 1 : 2;
      } else {
        uint32_t gv = gen0;
        for (int polls = 0; gv == gen0 && polls < kSpinLimit; ++polls) {
          __builtin_amdgcn_s_sleep(2);
          gv = (uint32_t)__hip_atomic_fetch_add(gen, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        flag = gv - gen0 == 1u ? 1 : 2;
      }
      merge_flag = flag;
    }
    __syncthreads();
    merge_share<D, NRG * KS * 64, NRG * 16>(a, g, row0, s, merge_flag == 2);
  }
}

template <int D, int NRG, int KS>
hipError_t launch_t(const ChunkAttnArgs& a, hipStream_t stream, bool* merged) {
  const int rows = a.q_len * a.G;
  const int tiles = (rows + NRG * 16 - 1) / (NRG * 16);
  const dim3 blocks(a.n_kv_heads * a.num_splits, tiles);
  const dim3 threads(NRG * KS * 64);
  const bool app = a.k_new != nullptr;
  if (a.pt != nullptr)
    return app ? launch_kernel(chunk_attn_kernel<D, NRG, KS, true, false, true>, blocks, threads, a, stream)
               : launch_kernel(chunk_attn_kernel<D, NRG, KS, true, false, false>, blocks, threads, a, stream);
  // the one-launch ring layer: counters given, few enough splits for the merge's registers,
  // (KV head, row tile) groups that divide evenly over the XCDs, and a grid that fits one
  // workgroup per compute unit (every workgroup of a group is resident while the others wait)
  const int64_t groups = (int64_t)a.n_kv_heads * tiles;
  if (a.tickets != nullptr && a.part_o != nullptr && a.num_splits > 1 &&
      a.num_splits <= kFuseMaxSplits && groups % kXcds == 0 &&
      groups * kTicketStride <= (int64_t)kTicketBytes && groups * a.num_splits <= a.fill_wgs) {
    *merged = true;
    const dim3 grid((unsigned)(groups * a.num_splits));
    return app ? launch_kernel(chunk_attn_kernel<D, NRG, KS, false, true, true>, grid, threads, a, stream)
               : launch_kernel(chunk_attn_kernel<D, NRG, KS, false, true, false>, grid, threads, a, stream);
  }
  return app ? launch_kernel(chunk_attn_kernel<D, NRG, KS, false, false, true>, blocks, threads, a, stream)
             : launch_kernel(chunk_attn_kernel<D, NRG, KS, false, false, false>, blocks, threads, a, stream);
}

// Tiles of 64 rows (blockIdx.y), two waves per row group (key halves).  Tiles of one split
// each read its chunks; a variant with more row groups per workgroup would need more registers
// than the register stages leave.  The tile is the smallest of 16, 32 and 64 rows whose grid
// still fits one round of one workgroup per compute unit (a smaller tile's workgroup takes a
// whole unit too, by its registers): a window layer runs 160 workgroups of 16 rows instead of
// 40 of 64, a pool context of 8,192 256 of 32 rows instead of 128; smaller tiles divide each
// workgroup's arithmetic per chunk, and the tiles of one split read the same chunks, after the
// first time from cache.  A grid of 132 workgroups keeps 64 rows (264 would take two rounds),
// and the long contexts keep them too, their 256 workgroups already filling the chip.
template <int D>
hipError_t launch_d(const ChunkAttnArgs& a, hipStream_t stream, bool* merged) {
  const int rows = a.q_len * a.G;
  const int64_t wgs = (int64_t)a.n_kv_heads * a.num_splits * ((rows + 63) / 64);
  if (4 * wgs <= a.fill_wgs) return launch_t<D, 1, 2>(a, stream, merged);
  if (2 * wgs <= a.fill_wgs) return launch_t<D, 2, 2>(a, stream, merged);
  return launch_t<D, 4, 2>(a, stream, merged);
}

}  // namespace

hipError_t launch_chunk_attn(const ChunkAttnArgs& a, hipStream_t stream, bool* merged) {
  *merged = false;
  if (a.q_len * a.G > kVerifyMaxRows) return launch_prefill_attn(a, stream);
  if (a.head_dim == 128) return launch_d<128>(a, stream, merged);
  return launch_d<64>(a, stream, merged);
}

}  // namespace rkv
