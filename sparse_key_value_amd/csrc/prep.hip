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
// (r % per_tok) * width in the input (in_ld elements per token).  The output row is the
// input row cut into segments of `seg` elements, each stored in `seg_ld` >= seg elements
// followed by zeros (seg_ld = seg: rows back to back, nothing padded); output row r starts at
// r * (width / seg) * seg_ld.  VEC: the input read four elements (16 bytes of fp32, 8 of bf16)
// per lane at a time, unpadded output only.  Q8 (VEC with 256-wide segments): also the fp8 copy
// of the output row (q8, same layout, one byte per element) and the fp32 norm of every segment
// (qn).
template <typename TI, typename TO, bool VEC, bool Q8 = false>
__global__ void __launch_bounds__(256) rownorm_kernel(const TI* __restrict__ in, TO* __restrict__ out,
                                                      int64_t rows, int width, int per_tok, int64_t in_ld, int norm,
                                                      float eps, int seg, int seg_ld, uint8_t* __restrict__ q8 = nullptr,
                                                      float* __restrict__ qn = nullptr) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const TI* src = in + (row / per_tok) * in_ld + (row % per_tok) * (int64_t)width;
  const int nseg = width / seg;
  TO* dst = out + row * (int64_t)nseg * seg_ld;
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
        if constexpr (sizeof(TI) == 4) {
          v[i] = *(const f32x4*)((const float*)src + i * 256 + lane * 4);
        } else {
          const uint2 p = *(const uint2*)((const uint16_t*)src + i * 256 + lane * 4);
          v[i] = f32x4{bf16_lo(p.x), bf16_hi(p.x), bf16_lo(p.y), bf16_hi(p.y)};
        }
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
    if constexpr (Q8) {
#pragma unroll
      for (int i = 0; i < MAXV; ++i) {
        if (i < nv) {
          const f32x4 w = v[i] * scale;
          *(uint32_t*)(q8 + row * (int64_t)width + i * 256 + lane * 4) = f32x4_to_fp8(w[0], w[1], w[2], w[3]);
          const float h = wave_sum_f32(w[0] * w[0] + w[1] * w[1] + w[2] * w[2] + w[3] * w[3]);
          if (lane == 0) qn[row * nv + i] = __fsqrt_rn(h);
        }
      }
    }
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
    if (seg == seg_ld) {
      for (int i = lane; i < width; i += 64) store_elem<TO>(dst, i, load_elem<TI>(src, i) * scale);
    } else {
      for (int i = lane; i < width; i += 64) store_elem<TO>(dst, (i / seg) * seg_ld + i % seg, load_elem<TI>(src, i) * scale);
      const int pad = seg_ld - seg;
      for (int i = lane; i < nseg * pad; i += 64) store_elem<TO>(dst, (i / pad) * seg_ld + seg + i % pad, 0.0f);
    }
  }
}

hipError_t launch_rownorm(const void* in, int in_is_f32, void* out, int out_dtype, int64_t rows, int width,
                          int norm, float eps, hipStream_t s, int per_tok, int64_t in_ld, int seg, int seg_ld,
                          uint8_t* q8, float* qn) {
  if (rows == 0) return hipSuccess;
  if (in_ld == 0) in_ld = (int64_t)per_tok * width;
  if (seg == 0) seg = seg_ld = width;
  dim3 grid((unsigned)((rows + 3) / 4));
  const bool vec = width % 256 == 0 && width <= 1024 && in_ld % 4 == 0 &&
                   ((uintptr_t)in & (in_is_f32 ? 15 : 7)) == 0 && seg == seg_ld;
#define PKM_RN(TI, TO, V)                                                                                          \
  rownorm_kernel<TI, TO, V><<<grid, 256, 0, s>>>((const TI*)in, (TO*)out, rows, width, per_tok, in_ld, norm, eps, seg, \
                                                 seg_ld)
  if (q8) {  // fp8 copy and segment norms with the bf16 rows: 256-wide segments
    if (!vec || seg != 256 || out_dtype != DT_BF16) {
      const hipError_t e =
          launch_rownorm(in, in_is_f32, out, out_dtype, rows, width, norm, eps, s, per_tok, in_ld, seg, seg_ld);
      if (e != hipSuccess) return e;
      return launch_fp8_rows(out, q8, qn, rows * (width / seg), seg_ld, nullptr, 1, s);
    }
    if (in_is_f32)
      rownorm_kernel<float, uint16_t, true, true><<<grid, 256, 0, s>>>((const float*)in, (uint16_t*)out, rows, width,
                                                                       per_tok, in_ld, norm, eps, seg, seg_ld, q8, qn);
    else
      rownorm_kernel<uint16_t, uint16_t, true, true><<<grid, 256, 0, s>>>(
          (const uint16_t*)in, (uint16_t*)out, rows, width, per_tok, in_ld, norm, eps, seg, seg_ld, q8, qn);
    return hipGetLastError();
  }
  if (in_is_f32) {
    if (out_dtype == DT_BF16) {
      if (vec) PKM_RN(float, uint16_t, true); else PKM_RN(float, uint16_t, false);
    } else {
      if (vec) PKM_RN(float, float, true); else PKM_RN(float, float, false);
    }
  } else {
    if (out_dtype == DT_BF16) {
      if (vec) PKM_RN(uint16_t, uint16_t, true); else PKM_RN(uint16_t, uint16_t, false);
    } else {
      PKM_RN(uint16_t, float, false);
    }
  }
#undef PKM_RN
  return hipGetLastError();
}

// One wave per row of d bf16 elements (d a multiple of 4): dst8 = e4m3 of the row, norms[row] =
// its fp32 norm (if norms).
__global__ void __launch_bounds__(256) fp8_rows_kernel(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst8,
                                                       float* __restrict__ norms, int64_t rows, int d) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* r = src + row * d;
  float ss = 0.f;
  for (int i = lane * 4; i < d; i += 256) {
    const uint2 p = *(const uint2*)(r + i);
    const float a = bf16_lo(p.x), b = bf16_hi(p.x), c = bf16_lo(p.y), e = bf16_hi(p.y);
    ss += a * a + b * b + c * c + e * e;
    *(uint32_t*)(dst8 + row * d + i) = f32x4_to_fp8(a, b, c, e);
  }
  ss = wave_sum_f32(ss);
  if (norms && lane == 0) norms[row] = __fsqrt_rn(ss);
}

// kmax[g] = the largest of norms[g * group .. g * group + group - 1]; one block per group.
__global__ void __launch_bounds__(256) group_max_kernel(const float* __restrict__ norms, int group,
                                                        float* __restrict__ kmax) {
  __shared__ float part[4];
  const float* p = norms + (int64_t)blockIdx.x * group;
  float m = 0.f;
  for (int i = threadIdx.x; i < group; i += 256) m = fmaxf(m, p[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, WAVE));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) kmax[blockIdx.x] = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
}

hipError_t launch_fp8_rows(const void* src, uint8_t* dst8, float* norms, int64_t rows, int d, float* kmax, int group,
                           hipStream_t s) {
  if (rows == 0) return hipSuccess;
  fp8_rows_kernel<<<dim3((unsigned)((rows + 3) / 4)), 256, 0, s>>>((const uint16_t*)src, dst8, norms, rows, d);
  if (kmax) group_max_kernel<<<dim3((unsigned)(rows / group)), 256, 0, s>>>(norms, group, kmax);
  return hipGetLastError();
}

// dst row r = src row r (width elements) followed by zeros up to ld elements; a capped grid
// loops over the rows * ld outputs.
template <typename T>
__global__ void __launch_bounds__(256) pad_rows_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t rows,
                                                       int width, int ld) {
  const int64_t total = rows * ld;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / ld;
    const int c = (int)(i - r * ld);
    dst[i] = c < width ? src[r * width + c] : T(0);
  }
}

hipError_t launch_pad_rows(const void* src, void* dst, int64_t rows, int width, int ld, int dtype, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows * ld + 255) / 256;
  const dim3 grid((unsigned)(blocks < ((int64_t)1 << 20) ? blocks : ((int64_t)1 << 20)));
  if (dtype == DT_BF16) pad_rows_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, rows, width, ld);
  else pad_rows_kernel<float><<<grid, 256, 0, s>>>((const float*)src, (float*)dst, rows, width, ld);
  return hipGetLastError();
}

}  // namespace pkm

namespace pkm {

// A grid of at most 2^20 blocks loops over the n elements (n can pass the 2^32 work-items of
// one launch: T * d_value).
__global__ void __launch_bounds__(256) convert_f32_kernel(const float* __restrict__ in, uint16_t* __restrict__ out,
                                                          int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out[i] = f32_to_bf16(in[i]);
}

// fp32 -> dtype (bf16 rounding, or a plain copy for fp32).
hipError_t launch_convert_f32(const float* in, void* out, int64_t n, int dtype, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (dtype == DT_F32) return hipMemcpyAsync(out, in, (size_t)n * 4, hipMemcpyDeviceToDevice, s);
  const int64_t blocks = (n + 255) / 256;
  convert_f32_kernel<<<dim3((unsigned)(blocks < ((int64_t)1 << 20) ? blocks : ((int64_t)1 << 20))), 256, 0, s>>>(
      in, (uint16_t*)out, n);
  return hipGetLastError();
}

}  // namespace pkm
