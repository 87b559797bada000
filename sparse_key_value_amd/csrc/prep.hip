// Elementwise and row-wise preparation kernels:
//  * transpose of a weight matrix into the K-contiguous layout the GEMM reads,
//  * the qk-norm fold of the sub-key codebooks (once, at create),
//  * the qk-norm of the query and its split into halves (every forward).
// qk-norm is RMSNorm with unit gain ("Memory Layers at Scale" digest, Memory+ block);
// the query is normalised over its whole per-head width, then split into a front and
// a back half ("Memory inside the model" overview, how it works).
#include "kernels.hpp"

namespace pkm {

// dst[c, r] = src[r, c] for a rows x cols matrix; 32 x 32 tiles staged through LDS.
template <typename T>
__global__ void __launch_bounds__(256) transpose_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                        int rows, int cols) {
  __shared__ T tile[32][33];
  const int bx = blockIdx.x * 32, by = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    int r = by + ty + i, c = bx + tx;
    if (r < rows && c < cols) tile[ty + i][tx] = src[(size_t)r * cols + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    int c = bx + ty + i, r = by + tx;
    if (r < rows && c < cols) dst[(size_t)c * rows + r] = tile[tx][ty + i];
  }
}

hipError_t launch_transpose(const void* src, void* dst, int rows, int cols, int dtype, hipStream_t s) {
  dim3 grid((cols + 31) / 32, (rows + 31) / 32);
  if (dtype == DT_BF16)
    transpose_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, rows, cols);
  else
    transpose_kernel<float><<<grid, 256, 0, s>>>((const float*)src, (float*)dst, rows, cols);
  return hipGetLastError();
}

template <typename T>
__device__ __forceinline__ float load_elem(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }

template <typename T>
__device__ __forceinline__ void store_elem(T* p, size_t i, float v);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, size_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }

// One wave per row of `width` elements: out = norm ? v / sqrt(mean(v^2) + eps) : v.
// Input element type TI (fp32 accumulator or stored dtype), output type TO.  Row r is
// element (r % per_tok) of token r / per_tok: it starts at (r / per_tok) * in_ld +
// (r % per_tok) * width in the input (in_ld elements per token) and at r * width in the
// output.  VEC: fp32 input read four elements (16 bytes) per lane at a time.
template <typename TI, typename TO, bool VEC>
__global__ void __launch_bounds__(256) rownorm_kernel(const TI* __restrict__ in, TO* __restrict__ out,
                                                      int64_t rows, int width, int per_tok, int64_t in_ld, int norm,
                                                      float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const TI* src = in + (row / per_tok) * in_ld + (row % per_tok) * (int64_t)width;
  TO* dst = out + row * width;
  float scale = 1.0f;
  if constexpr (VEC) {
    // width is a multiple of 256: every lane holds width / 256 groups of four
    constexpr int MAXV = 4;  // width <= 1024
    f32x4 v[MAXV];
    const int nv = width / 256;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      if (i < nv) {
        v[i] = *(const f32x4*)((const float*)src + i * 256 + lane * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += v[i][e] * v[i][e];
      }
    }
    if (norm) {
      ss = wave_sum_f32(ss);
      scale = 1.0f / __fsqrt_rn(ss / (float)width + eps);
    }
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
      if (i < nv)
#pragma unroll
        for (int e = 0; e < 4; ++e) store_elem<TO>(dst, i * 256 + lane * 4 + e, v[i][e] * scale);
  } else {
    if (norm) {
      float ss = 0.f;
      for (int i = lane; i < width; i += 64) {
        float v = load_elem<TI>(src, i);
        ss += v * v;
      }
      ss = wave_sum_f32(ss);
      scale = 1.0f / __fsqrt_rn(ss / (float)width + eps);
    }
    for (int i = lane; i < width; i += 64) store_elem<TO>(dst, i, load_elem<TI>(src, i) * scale);
  }
}

hipError_t launch_rownorm(const void* in, int in_is_f32, void* out, int out_dtype, int64_t rows, int width,
                          int norm, float eps, hipStream_t s, int per_tok, int64_t in_ld) {
  if (rows == 0) return hipSuccess;
  if (in_ld == 0) in_ld = (int64_t)per_tok * width;
  dim3 grid((unsigned)((rows + 3) / 4));
  const bool vec = in_is_f32 && width % 256 == 0 && width <= 1024 && in_ld % 4 == 0 && ((uintptr_t)in & 15) == 0;
#define PKM_RN(TI, TO, V) \
  rownorm_kernel<TI, TO, V><<<grid, 256, 0, s>>>((const TI*)in, (TO*)out, rows, width, per_tok, in_ld, norm, eps)
  if (in_is_f32) {
    if (out_dtype == DT_BF16) {
      if (vec) PKM_RN(float, uint16_t, true); else PKM_RN(float, uint16_t, false);
    } else {
      if (vec) PKM_RN(float, float, true); else PKM_RN(float, float, false);
    }
  } else {
    if (out_dtype == DT_BF16) PKM_RN(uint16_t, uint16_t, false);
    else PKM_RN(uint16_t, float, false);
  }
#undef PKM_RN
  return hipGetLastError();
}

}  // namespace pkm

namespace pkm {

__global__ void __launch_bounds__(256) convert_f32_kernel(const float* __restrict__ in, uint16_t* __restrict__ out,
                                                          int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = f32_to_bf16(in[i]);
}

// fp32 -> dtype (bf16 rounding, or a plain copy for fp32).
hipError_t launch_convert_f32(const float* in, void* out, int64_t n, int dtype, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (dtype == DT_F32) return hipMemcpyAsync(out, in, (size_t)n * 4, hipMemcpyDeviceToDevice, s);
  convert_f32_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(in, (uint16_t*)out, n);
  return hipGetLastError();
}

}  // namespace pkm
