// Shared device helpers of the product-key memory kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// ---- bf16 <-> fp32 ------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 with round-to-nearest-even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- ordered selection keys ---------------------------------------------------
// A candidate (score, index) becomes one 64-bit key whose unsigned order is the
// selection order: higher score first, then lower index.  The score part is the
// usual order-preserving map of IEEE floats onto unsigned integers (flip all
// bits of negatives, set the sign bit of non-negatives), after mapping -0 to +0;
// the index part is stored complemented so that a lower index is a larger key.
// Key 0 is below every real key and marks an empty slot.

__device__ __forceinline__ uint32_t ord_score(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float score_of_ord(uint32_t o) {
  uint32_t b = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(b);
}
__device__ __forceinline__ uint64_t make_key(float s, uint32_t idx) {
  return ((uint64_t)ord_score(s) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)k; }
__device__ __forceinline__ float key_score(uint64_t k) { return score_of_ord((uint32_t)(k >> 32)); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m, WAVE);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, WAVE);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl((uint32_t)v, src, WAVE);
  uint32_t hi = __shfl((uint32_t)(v >> 32), src, WAVE);
  return ((uint64_t)hi << 32) | lo;
}

// The 64-bit value of lane `src` (a wave-uniform lane index), broadcast to every lane.
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// Sort one key per lane across the 64 lanes of a wave, descending (lane 0 = largest).
// Bitonic network (Batcher 1968): log2(64) * (log2(64) + 1) / 2 = 21 compare-exchange steps.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t key, int lane) {
#pragma unroll
  for (int size = 2; size <= WAVE; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      uint64_t other = shfl_xor_u64(key, stride);
      bool desc_block = (lane & size) == 0;
      bool lower = (lane & stride) == 0;
      bool take_max = (desc_block == lower);
      uint64_t mx = key > other ? key : other;
      uint64_t mn = key > other ? other : key;
      key = take_max ? mx : mn;
    }
  }
  return key;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 1; m < WAVE; m <<= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 1; m < WAVE; m <<= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace pkm
