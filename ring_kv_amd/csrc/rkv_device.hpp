// Device helpers for the gfx950 (CDNA4) kernels of libring_kv.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kChunk = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even f32 pair -> packed bf16 (low half = a); gfx950 has this in hardware.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// 16x16x32 bf16 MFMA: lane l supplies row (l & 15) of A and column (l & 15) of B, each as
// 8 consecutive k-values of k-group (l >> 4); C lane l holds rows 4*(l>>4)+0..3 of column
// (l & 15).  A and B use the same k-group mapping, so any assignment of reduction indices to
// (group, slot) pairs gives the same sum as long as A and B agree on it.
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_xor(float v, int mask) { return __shfl_xor(v, mask, kWave); }

__device__ __forceinline__ int64_t imax64(int64_t a, int64_t b) { return a > b ? a : b; }
__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global memory, which
// the backend lowers to a wait for every vector-memory load in flight: it would drain the
// KV prefetch at every barrier.  LDS traffic is all these barriers have to order.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup order that keeps consecutive logical blocks on one XCD: the dispatcher deals
// blocks round-robin over the 8 XCDs, so physical block b runs on XCD b % 8.
__device__ __forceinline__ int xcd_block(int b, int nb) {
  return (nb & 7) ? b : (b & 7) * (nb >> 3) + (b >> 3);
}

// ---- log-sum-exp merge of split partials ----------------------------------------------------
// Each output element sums, for each split group k = s mod SG, the group's splits in order of s,
// then the SG group sums in order of k (SG = 1024 / D: the merge kernel's 256 threads hold D / 4
// four-element columns per group).  Every merge path here uses this grouping and these helpers,
// so all of them give the same bits.
template <int D>
constexpr int merge_groups() { return 1024 / D; }

// Split s's weight exp(lse_s - Mu) (an lse of -inf, a split that saw no key of the row, weighs
// 0; a NaN lse weighs NaN and the row comes out NaN), and its term added to the running sums.
__device__ __forceinline__ float merge_weight(float ls, float Mu) {
  return ls != -INFINITY ? expf(ls - Mu) : 0.f;
}
__device__ __forceinline__ void merge_add(f32x4& acc, float& L, f32x4 o, float w) {
  acc += o * w;
  L += w;
}
__device__ __forceinline__ void merge_term(f32x4& acc, float& L, f32x4 o, float ls, float Mu) {
  merge_add(acc, L, o, merge_weight(ls, Mu));
}
__device__ __forceinline__ f32x4 merge_out(f32x4 acc, float Lt) {
  return Lt != 0.f ? acc * (1.f / Lt) : f32x4{0.f, 0.f, 0.f, 0.f};
}
__device__ __forceinline__ float merge_lse(float M, float Lt) {
  return Lt != 0.f ? M + logf(Lt) : -INFINITY;
}

}  // namespace rkv
