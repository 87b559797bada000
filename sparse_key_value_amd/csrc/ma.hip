// Memory Attention token-memory values (summary of "Memory Attention": how it works --
// V = K + RMSNorm per key/value head of E[s]; how it differs -- the norm folded into the
// table at inference, so V = K + E_bar[s]) and their C entry points.
//
// ma_fold_table runs once per table: one thread per (row, head) slice reads the slice
// with 16-byte loads, forms the fp32 mean square and writes the scaled slice.
// ma_values is the lookup itself, a k = 1 weight-1 EmbeddingBag fused with the add: one
// thread per 16-byte slice of a token, reading the slice of K and of the token's table
// row (plain loads: a 32,000-row table of 4 KiB rows mostly stays in the 256 MB
// last-level cache) and writing the slice of V.
#include "../../include/ma.h"
#include "abi.hpp"
#include "checks.hpp"
#include "common.hpp"

namespace pkm {

namespace {

template <int EB>
struct Vec;
template <>
struct Vec<2> {
  static constexpr int E = 8;
  __device__ static __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16_lo(v[e]);
      f[2 * e + 1] = bf16_hi(v[e]);
    }
  }
  __device__ static __forceinline__ u32x4 pack(const float* f) {
    u32x4 p;
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = (uint32_t)f32_to_bf16(f[2 * e]) | ((uint32_t)f32_to_bf16(f[2 * e + 1]) << 16);
    return p;
  }
};
template <>
struct Vec<4> {
  static constexpr int E = 4;
  __device__ static __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(v[e]);
  }
  __device__ static __forceinline__ u32x4 pack(const float* f) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
  }
};

// Slice (row, head) = i of the fold.
template <int EB>
__device__ __forceinline__ void fold_one(const uint8_t* __restrict__ E, int slices, int head_vecs, int n_heads,
                                         const float* __restrict__ gain, float eps, uint8_t* __restrict__ out,
                                         int64_t i) {
  using V = Vec<EB>;
  constexpr int NE = V::E;
  const int64_t row = i / n_heads;
  const int h = (int)(i - row * n_heads);
  const uint8_t* src = E + ((size_t)row * slices + (size_t)h * head_vecs) * 16;
  uint8_t* dst = out + ((size_t)row * slices + (size_t)h * head_vecs) * 16;
  float ss = 0.f;
  for (int v = 0; v < head_vecs; ++v) {
    float f[NE];
    V::unpack(*(const u32x4*)(src + (size_t)v * 16), f);
#pragma unroll
    for (int x = 0; x < NE; ++x) ss = __builtin_fmaf(f[x], f[x], ss);
  }
  const float rs = 1.0f / __fsqrt_rn(ss / (float)(head_vecs * NE) + eps);
  for (int v = 0; v < head_vecs; ++v) {
    float f[NE];
    V::unpack(*(const u32x4*)(src + (size_t)v * 16), f);
    const int c0 = (h * head_vecs + v) * NE;
#pragma unroll
    for (int x = 0; x < NE; ++x) f[x] = gain ? (f[x] * rs) * gain[c0 + x] : f[x] * rs;
    *(u32x4*)(dst + (size_t)v * 16) = V::pack(f);
  }
}

// One thread per (row, head) slice; a capped grid loops.
template <int EB>
__global__ void __launch_bounds__(256) fold_kernel(const uint8_t* __restrict__ E, int64_t vocab, int slices,
                                                   int head_vecs, int n_heads, const float* __restrict__ gain,
                                                   float eps, uint8_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < vocab * n_heads; i += (int64_t)gridDim.x * 256)
    fold_one<EB>(E, slices, head_vecs, n_heads, gain, eps, out, i);
}

// Slice i = t * slices + s of V = K + E_bar[ids[t]].
template <int EB>
__device__ __forceinline__ void value_one(const uint8_t* __restrict__ Ebar, int64_t vocab, int slices,
                                          const int32_t* __restrict__ ids, const uint8_t* __restrict__ K,
                                          uint8_t* __restrict__ Vout, int64_t i) {
  using V = Vec<EB>;
  constexpr int NE = V::E;
  const int64_t t = i / slices;
  const int s = (int)(i - t * slices);
  const int32_t id = ids[t];
  float k[NE];
  V::unpack(__builtin_nontemporal_load((const u32x4*)(K + (size_t)i * 16)), k);
  if (id >= 0 && (int64_t)id < vocab) {
    float e[NE];
    V::unpack(*(const u32x4*)(Ebar + ((size_t)id * slices + s) * 16), e);
#pragma unroll
    for (int x = 0; x < NE; ++x) k[x] += e[x];
  }
  __builtin_nontemporal_store(V::pack(k), (u32x4*)(Vout + (size_t)i * 16));
}

// One thread per 16-byte slice of a token; a capped grid loops.
template <int EB>
__global__ void __launch_bounds__(256) values_kernel(const uint8_t* __restrict__ Ebar, int64_t vocab, int slices,
                                                     const int32_t* __restrict__ ids, int64_t T,
                                                     const uint8_t* __restrict__ K, uint8_t* __restrict__ Vout) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < T * slices; i += (int64_t)gridDim.x * 256)
    value_one<EB>(Ebar, vocab, slices, ids, K, Vout, i);
}

int device_ok() {
  static int state[64] = {};
  int dev = 0;
  PKM_HIP(hipGetDevice(&dev));
  if (dev >= 0 && dev < 64 && state[dev] == 1) return PKM_OK;
  const int rc = pkm_abi::check_device();
  if (rc == PKM_OK && dev >= 0 && dev < 64) state[dev] = 1;
  return rc;
}

}  // namespace

}  // namespace pkm

extern "C" {

int ma_fold_table(const void* E, int64_t vocab, int32_t d_v, int32_t n_heads, const float* gain, float eps,
                  int32_t dtype, void* E_bar, void* stream) {
  using pkm_abi::fail;
  const std::string why = pkm::check_ma_fold(vocab, d_v, n_heads, eps, dtype);
  if (!why.empty()) return fail(PKM_EINVAL, "%s", why.c_str());
  const int eb = dtype == PKM_BF16 ? 2 : 4;
  if (vocab == 0) return PKM_OK;
  if (!E || !E_bar) return fail(PKM_EINVAL, "E and E_bar must not be NULL");
  if ((((uintptr_t)E | (uintptr_t)E_bar) & 15) != 0) return fail(PKM_EINVAL, "E and E_bar must be 16-byte aligned");
  int rc = pkm::device_ok();
  if (rc != PKM_OK) return rc;
  const int slices = d_v * eb / 16, head_vecs = slices / n_heads;
  const int64_t n = vocab * n_heads;
  const dim3 grid((unsigned)((n + 255) / 256 < ((int64_t)1 << 20) ? (n + 255) / 256 : ((int64_t)1 << 20)));
  hipStream_t s = (hipStream_t)stream;
  if (dtype == PKM_BF16)
    PKM_LAUNCH((pkm::fold_kernel<2><<<grid, 256, 0, s>>>((const uint8_t*)E, vocab, slices, head_vecs, n_heads, gain,
                                                         eps, (uint8_t*)E_bar), hipGetLastError()));
  else
    PKM_LAUNCH((pkm::fold_kernel<4><<<grid, 256, 0, s>>>((const uint8_t*)E, vocab, slices, head_vecs, n_heads, gain,
                                                         eps, (uint8_t*)E_bar), hipGetLastError()));
  return PKM_OK;
}

int ma_values(const void* E_bar, int64_t vocab, int32_t d_v, int32_t dtype, const int32_t* ids, int64_t T,
              const void* K, void* V, void* stream) {
  using pkm_abi::fail;
  const std::string why = pkm::check_ma_values(vocab, d_v, dtype, T);
  if (!why.empty()) return fail(PKM_EINVAL, "%s", why.c_str());
  const int eb = dtype == PKM_BF16 ? 2 : 4;
  if (T == 0) return PKM_OK;
  if (!E_bar || !ids || !K || !V) return fail(PKM_EINVAL, "E_bar, ids, K and V must not be NULL");
  if ((((uintptr_t)E_bar | (uintptr_t)K | (uintptr_t)V) & 15) != 0)
    return fail(PKM_EINVAL, "E_bar, K and V must be 16-byte aligned");
  int rc = pkm::device_ok();
  if (rc != PKM_OK) return rc;
  const int slices = d_v * eb / 16;
  const int64_t n = T * slices;
  const dim3 grid((unsigned)((n + 255) / 256 < ((int64_t)1 << 20) ? (n + 255) / 256 : ((int64_t)1 << 20)));
  hipStream_t s = (hipStream_t)stream;
  if (dtype == PKM_BF16)
    PKM_LAUNCH((pkm::values_kernel<2><<<grid, 256, 0, s>>>((const uint8_t*)E_bar, vocab, slices, ids, T,
                                                           (const uint8_t*)K, (uint8_t*)V), hipGetLastError()));
  else
    PKM_LAUNCH((pkm::values_kernel<4><<<grid, 256, 0, s>>>((const uint8_t*)E_bar, vocab, slices, ids, T,
                                                           (const uint8_t*)K, (uint8_t*)V), hipGetLastError()));
  return PKM_OK;
}

}  // extern "C"
