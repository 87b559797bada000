// Shared device helpers of the product-key memory kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

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

// Four fp32 values to OCP fp8 e4m3 (round to nearest even), packed in one word, first value
// in the low byte.  The conversion turns values beyond the format's 448 into NaN, so they are
// clamped to +-448 first.
__device__ __forceinline__ uint32_t f32x4_to_fp8(float a, float b, float c, float d) {
  auto cl = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
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

// The other half of the wave (lane l ^ 32) on gfx950's v_permlane32_swap, a VALU op, rather
// than ds_bpermute (an LDS round trip, whose wait also waits for every LDS read in flight).
// swap32(x) = {r0, r1} with r0 = x in lanes 0-31 and lane l - 32's x in lanes 32-63, r1 = lane
// l + 32's x in lanes 0-31 and x in lanes 32-63: every lane holds its own and its partner's.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ int add_xor32(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return (int)(r[0] + r[1]);
}

// x of lane l ^ s for s = 1, 2, 4, ..., 32 (a constant once the caller's loop is unrolled), on
// the VALU rather than through ds_bpermute: DPP quad permutes for 1 and 2, a row half-mirror
// (l ^ 7) or row mirror (l ^ 15) followed by a quad reversal (l ^ 3) or half-mirror for 4 and
// 8, and v_permlane16_swap / v_permlane32_swap for 16 and 32 (each returns a lane's own value
// and its partner's, in an order set by the lane's bit s).
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t x, int s) {
  constexpr int QXOR1 = 0xB1, QXOR2 = 0x4E, QREV = 0x1B, ROW_MIRROR = 0x140, ROW_HALF_MIRROR = 0x141;
  switch (s) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, QXOR1, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, QXOR2, 0xF, 0xF, false);
    case 4: {
      const int t = __builtin_amdgcn_mov_dpp((int)x, ROW_HALF_MIRROR, 0xF, 0xF, false);
      return (uint32_t)__builtin_amdgcn_mov_dpp(t, QREV, 0xF, 0xF, false);
    }
    case 8: {
      const int t = __builtin_amdgcn_mov_dpp((int)x, ROW_MIRROR, 0xF, 0xF, false);
      return (uint32_t)__builtin_amdgcn_mov_dpp(t, ROW_HALF_MIRROR, 0xF, 0xF, false);
    }
    case 16: {
      const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
      return (__lane_id() & 16) ? r[0] : r[1];
    }
    case 32: {
      const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
      return (__lane_id() & 32) ? r[0] : r[1];
    }
    default: return (uint32_t)__shfl_xor((int)x, s, WAVE);
  }
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = xor_lane_u32((uint32_t)v, m);
  const uint32_t hi = xor_lane_u32((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
// The lanes of a wave whose bit s (a power of two) is clear, as a 64-bit lane mask; and a
// lane's bit of a wave-uniform mask, read from the mask itself (no per-lane arithmetic: the
// select that uses it takes the mask as its condition).
__device__ __forceinline__ constexpr uint64_t lanes_bit_clear(int s) {
  return s == 1 ? 0x5555555555555555ull : s == 2 ? 0x3333333333333333ull : s == 4 ? 0x0F0F0F0F0F0F0F0Full
       : s == 8 ? 0x00FF00FF00FF00FFull : s == 16 ? 0x0000FFFF0000FFFFull : s == 32 ? 0x00000000FFFFFFFFull : ~0ull;
}
__device__ __forceinline__ bool lane_in(uint64_t mask) { return __builtin_amdgcn_inverse_ballot_w64(mask); }

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
      const uint64_t other = shfl_xor_u64(key, stride);
      // keep the larger where bit `size` and bit `stride` of the lane agree
      const bool take_max = lane_in(~(lanes_bit_clear(size) ^ lanes_bit_clear(stride)));
      key = (key > other) == take_max ? key : other;  // one compare, two selects
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
  for (int m = 1; m < WAVE; m <<= 1) v += __uint_as_float(xor_lane_u32(__float_as_uint(v), m));
  return v;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace pkm
