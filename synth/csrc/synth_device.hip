// Input-generation and bandwidth-reference kernels (benchmark and test harness only;
// not part of the product-key memory path).
//
//  * synth_fill_values: the row-addressable value table, bit-identical to the host
//    generator in synth/inputs.py:
//        seed_V = splitmix64((seed << 8) | tid)     (tid 6: the value table)
//        u      = splitmix64(seed_V ^ (row * d_v + col))
//        S      = sum of the four 16-bit limbs of u
//        v      = (S - 131070) * 0x1.1bc779ef9b324p-21      (IEEE double)
//        stored = float(v), or bf16(float(v)) with round-to-nearest-even
//    splitmix64: Steele, Lea & Flood, "Fast splittable pseudorandom number
//    generators", OOPSLA 2014.
//  * synth_stream_read: reads a buffer once with 16-byte nontemporal loads (the
//    streaming-read ceiling of the HBM).
//  * synth_copy: a plain 16-byte copy kernel of known size, used to calibrate the
//    HBM byte counters.
//  * synth_row_read: reads the rows a list of bags names, with the lane layout of a
//    weighted bag gather (one 16-byte column slice per lane, 16 rows in flight), and
//    only XORs them: the read rate of those random rows with no arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __host__ __forceinline__ uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float gen_value(uint64_t sv, uint64_t ctr) {
  const uint64_t u = splitmix64(sv ^ ctr);
  const int64_t s = (int64_t)(u & 0xFFFF) + (int64_t)((u >> 16) & 0xFFFF) + (int64_t)((u >> 32) & 0xFFFF) +
                    (int64_t)(u >> 48);
  const double v = (double)(s - 131070) * 0x1.1bc779ef9b324p-21;
  return __double2float_rn(v);
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// one thread per 16 bytes of output
__global__ void fill_values_kernel(uint8_t* __restrict__ dst, int64_t row0, int64_t n_rows, int d_v, int bf16,
                                   uint64_t sv) {
  const int per = bf16 ? 8 : 4;
  const int64_t units_per_row = d_v / per;
  const int64_t total = n_rows * units_per_row;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = row0 + u / units_per_row;
    const int64_t c0 = (u % units_per_row) * per;
    const uint64_t base = (uint64_t)r * (uint64_t)d_v + (uint64_t)c0;
    u32x4 out;
    if (bf16) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        out[e] = bf16_rne(gen_value(sv, base + 2 * e)) | (bf16_rne(gen_value(sv, base + 2 * e + 1)) << 16);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = __float_as_uint(gen_value(sv, base + e));
    }
    *(u32x4*)(dst + ((uint64_t)r * d_v + c0) * (bf16 ? 2 : 4)) = out;
  }
}

__global__ void stream_read_kernel(const u32x4* __restrict__ p, int64_t n16, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x) {
    u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads live; practically never taken
}

__global__ void copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = __builtin_nontemporal_load(src + i);
}

// Bag b's rows idx[b * bag ..][0, bag): lane slice `col` of each, XORed, one 16-byte store per lane
// and bag into out[b * row_vecs + col]; indices outside [0, n_rows) read row 0.
__global__ void __launch_bounds__(256) row_read_kernel(const uint8_t* __restrict__ table, int64_t n_rows,
                                                       int row_vecs, int tpr, int bpb,
                                                       const int32_t* __restrict__ idx, int64_t n_bags, int bag,
                                                       u32x4* __restrict__ out) {
  const int g = threadIdx.x / tpr;
  const int col = blockIdx.y * tpr + (threadIdx.x - g * tpr);
  if (g >= bpb || col >= row_vecs) return;
  const size_t rb = (size_t)row_vecs * 16;
  auto slice = [&](int32_t r) {
    r = (uint64_t)(int64_t)r < (uint64_t)n_rows ? r : 0;
    return __builtin_nontemporal_load((const u32x4*)(table + (size_t)r * rb) + col);
  };
  for (int64_t b = (int64_t)blockIdx.x * bpb + g; b < n_bags; b += (int64_t)gridDim.x * bpb) {
    const int32_t* bi = idx + b * bag;
    u32x4 acc = {0u, 0u, 0u, 0u};
    int j = 0;
    for (; j + 16 <= bag; j += 16) {
      u32x4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = slice(bi[j + u]);
#pragma unroll
      for (int u = 0; u < 16; ++u) acc ^= v[u];
    }
    for (; j < bag; ++j) acc ^= slice(bi[j]);
    __builtin_nontemporal_store(acc, out + b * row_vecs + col);
  }
}

extern "C" {

// Fill rows [row0, row0 + n_rows) of a [*, d_v] table at `table` (device pointer to row 0)
// from the stream of tensor id `tid`.  dtype 0 = fp32, 1 = bf16.  Returns 0 or a
// hipError_t code.
int synth_fill_table(void* table, int64_t row0, int64_t n_rows, int32_t d_v, int32_t dtype, uint64_t seed,
                     uint32_t tid, void* stream) {
  const int per = dtype == 1 ? 8 : 4;
  if (!table || n_rows < 0 || row0 < 0 || d_v <= 0 || d_v % per != 0 || tid > 255) return (int)hipErrorInvalidValue;
  if (n_rows == 0) return 0;
  const uint64_t sv = splitmix64((seed << 8) | tid);
  fill_values_kernel<<<8192, 256, 0, (hipStream_t)stream>>>((uint8_t*)table, row0, n_rows, d_v, dtype == 1, sv);
  return (int)hipGetLastError();
}

// The value table of the product-key memory: tensor id 6.
int synth_fill_values(void* table, int64_t row0, int64_t n_rows, int32_t d_v, int32_t dtype, uint64_t seed,
                      void* stream) {
  return synth_fill_table(table, row0, n_rows, d_v, dtype, seed, 6u, stream);
}

int synth_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid, void* stream) {
  if (!buf || !sink || bytes < 16 || grid < 1) return (int)hipErrorInvalidValue;
  stream_read_kernel<<<grid, 256, 0, (hipStream_t)stream>>>((const u32x4*)buf, bytes / 16, sink);
  return (int)hipGetLastError();
}

int synth_copy(void* dst, const void* src, int64_t bytes, int32_t grid, void* stream) {
  if (!dst || !src || bytes < 16 || grid < 1) return (int)hipErrorInvalidValue;
  copy_kernel<<<grid, 256, 0, (hipStream_t)stream>>>((u32x4*)dst, (const u32x4*)src, bytes / 16);
  return (int)hipGetLastError();
}

// out: n_bags x row_bytes bytes.  row_bytes: a multiple of 16.
int synth_row_read(const void* table, int64_t n_rows, int64_t row_bytes, const int32_t* idx, int64_t n_bags,
                   int32_t bag, void* out, void* stream) {
  if (!table || !idx || !out || n_rows < 1 || row_bytes < 16 || row_bytes % 16 != 0 || n_bags < 0 || bag < 1)
    return (int)hipErrorInvalidValue;
  if (n_bags == 0) return 0;
  const int row_vecs = (int)(row_bytes / 16);
  const int tpr = row_vecs < 256 ? row_vecs : 256, bpb = 256 / tpr;
  const int64_t cols = (row_vecs + tpr - 1) / tpr;
  if (cols > 65535) return (int)hipErrorInvalidValue;
  const int64_t groups = (n_bags + bpb - 1) / bpb, cap = ((int64_t)1 << 22) / cols;
  const dim3 grid((unsigned)(groups < cap ? groups : (cap > 0 ? cap : 1)), (unsigned)cols);
  row_read_kernel<<<grid, bpb * tpr, 0, (hipStream_t)stream>>>((const uint8_t*)table, n_rows, row_vecs, tpr, bpb, idx,
                                                              n_bags, bag, (u32x4*)out);
  return (int)hipGetLastError();
}

}  // extern "C"
