// Weighted EmbeddingBag gather-reduce over the value table.
//
// y[b, :] = sum over j of w[b, j] * table[idx[b, j], :]   ("Memory Layers at Scale"
// digest, parallel EmbeddingBag: the memory read is an EmbeddingBag and is bound by
// memory bandwidth, not FLOPs).  In the forward a bag is one token's H*k selected
// rows with their softmax weights (core idea: weighted sum of the top-k values).
// With the Memory+ gate (digest, Memory+ block) the kernel also applies the gate's
// elementwise part, g = y * silu(z) with z = x W1 computed beforehand (in the stored type),
// and writes g in the table's type instead of y in fp32: the fp32 y never reaches HBM.  Writes mixed
// into this read stream cost far more than their bytes (128 MiB of fp32 y slowed the
// 8.6 GB gather by about 16% on MI355X), while reading z costs about its bytes.
//
// Design for gfx950: every lane owns one 16-byte column slice of a row, so one row
// read by a group of lanes is one fully coalesced burst; a bag's indices and weights
// are wave-uniform and come through the scalar cache; UNROLL rows are put in flight
// before any is consumed (the table is far larger than the caches, so the loads are
// nontemporal); accumulation is fp32 in a fixed order, with no atomics, so results
// are bitwise reproducible.
#include "kernels.hpp"

namespace pkm {

template <int EB>
struct VecTraits;
template <>
struct VecTraits<2> {  // bf16: 8 elements per 16 bytes
  static constexpr int E = 8;
  __device__ static __forceinline__ void fma(float* acc, u32x4 v, float w) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = __builtin_fmaf(w, bf16_lo(v[e]), acc[2 * e]);
      acc[2 * e + 1] = __builtin_fmaf(w, bf16_hi(v[e]), acc[2 * e + 1]);
    }
  }
};
template <>
struct VecTraits<4> {  // fp32: 4 elements per 16 bytes
  static constexpr int E = 4;
  __device__ static __forceinline__ void fma(float* acc, u32x4 v, float w) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, __uint_as_float(v[e]), acc[e]);
  }
};

template <int EB, int UNROLL, int ZB>
__device__ __forceinline__ void gather_bag(const uint8_t* __restrict__ table, int64_t n_rows, int row_vecs, int col,
                                           const int32_t* __restrict__ idx, const float* __restrict__ w, int64_t b,
                                           int bag, void* __restrict__ y, int y_f32, const void* __restrict__ z,
                                           int64_t z_ld);

// Block = BAGS_PER_BLOCK groups of TPR lanes; group g handles bags blockIdx.x*BPB+g,
// then + gridDim.x*BPB, ... (one block per group of bags up to a grid cap), and the
// 16-byte column slices [blockIdx.y*TPR, blockIdx.y*TPR + TPR) of their rows.
template <int EB, int UNROLL, bool UNIFORM, int ZB>
__global__ void __launch_bounds__(256) gather_kernel(const uint8_t* __restrict__ table, int64_t n_rows,
                                                     int row_vecs, int tpr, int bags_per_block,
                                                     const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                     int64_t n_bags, int bag, void* __restrict__ y, int y_f32,
                                                     const void* __restrict__ z, int64_t z_ld) {
  int g = threadIdx.x / tpr;
  if (UNIFORM) g = __builtin_amdgcn_readfirstlane(g);
  const int col = blockIdx.y * tpr + (threadIdx.x - g * tpr);  // 16-byte slice index in the row
  if (g >= bags_per_block || col >= row_vecs) return;
  for (int64_t b = (int64_t)blockIdx.x * bags_per_block + g; b < n_bags; b += (int64_t)gridDim.x * bags_per_block)
    gather_bag<EB, UNROLL, ZB>(table, n_rows, row_vecs, col, idx, w, b, bag, y, y_f32, z, z_ld);
}

template <int EB, int UNROLL, int ZB>
__device__ __forceinline__ void gather_bag(const uint8_t* __restrict__ table, int64_t n_rows, int row_vecs, int col,
                                           const int32_t* __restrict__ idx, const float* __restrict__ w, int64_t b,
                                           int bag, void* __restrict__ y, int y_f32, const void* __restrict__ z,
                                           int64_t z_ld) {
  using VT = VecTraits<EB>;
  constexpr int E = VT::E;
  const int32_t* bi = idx + b * bag;
  const float* bw = w + b * bag;
  const size_t row_bytes = (size_t)row_vecs * 16;
  const uint8_t* base = table + (size_t)col * 16;

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;

  int j = 0;
  for (; j + UNROLL <= bag; j += UNROLL) {
    u32x4 v[UNROLL];
    float wt[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      int32_t r = bi[j + u];
      bool ok = (uint64_t)(int64_t)r < (uint64_t)n_rows;
      wt[u] = ok ? bw[j + u] : 0.f;
      r = ok ? r : 0;
      v[u] = __builtin_nontemporal_load((const u32x4*)(base + (size_t)r * row_bytes));
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) VT::fma(acc, v[u], wt[u]);
  }
  for (; j < bag; ++j) {
    int32_t r = bi[j];
    bool ok = (uint64_t)(int64_t)r < (uint64_t)n_rows;
    float wt = ok ? bw[j] : 0.f;
    r = ok ? r : 0;
    u32x4 v = __builtin_nontemporal_load((const u32x4*)(base + (size_t)r * row_bytes));
    VT::fma(acc, v, wt);
  }

  const int64_t dim = (int64_t)row_vecs * E;
  const int64_t o = b * dim + (int64_t)col * E;
  if constexpr (ZB != 0) {
    // g = y * silu(z), stored in the table's type; z in fp32 (ZB = 4) or bf16 (ZB = 2, with bf16
    // values): the lane's E elements of z in 16-byte loads when every z row is 16-byte aligned,
    // else (ZB < 0) in 4-byte loads (z rows are always 4-byte aligned)
    if constexpr (ZB == 4 || ZB == -4) {
      const float* zr = (const float*)z + b * z_ld + (int64_t)col * E;
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        f32x4 zz;
        if constexpr (ZB == 4) {
          zz = __builtin_nontemporal_load((const f32x4*)(zr + e));
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x) zz[x] = __builtin_nontemporal_load(zr + e + x);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[e + x] = acc[e + x] * silu_f32(zz[x]);
      }
    } else {
      static_assert((ZB == 2 || ZB == -2) && EB == 2, "a bf16 z goes with bf16 values");
      const uint16_t* zr = (const uint16_t*)z + b * z_ld + (int64_t)col * E;
      u32x4 zz;
      if constexpr (ZB == 2) {
        zz = __builtin_nontemporal_load((const u32x4*)zr);
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x) zz[x] = __builtin_nontemporal_load((const uint32_t*)zr + x);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        acc[2 * x] = acc[2 * x] * silu_f32(bf16_lo(zz[x]));
        acc[2 * x + 1] = acc[2 * x + 1] * silu_f32(bf16_hi(zz[x]));
      }
    }
    if constexpr (EB == 2) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pk[e] = (uint32_t)f32_to_bf16(acc[2 * e]) | ((uint32_t)f32_to_bf16(acc[2 * e + 1]) << 16);
      __builtin_nontemporal_store(pk, (u32x4*)((uint16_t*)y + o));
    } else {
      __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, (f32x4*)((float*)y + o));
    }
    return;
  }
  // outputs are streamed (nontemporal stores): they are not read again by this kernel
  if (y_f32) {
    float* yo = (float*)y + o;
#pragma unroll
    for (int e = 0; e < E; e += 4)
      __builtin_nontemporal_store(f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]}, (f32x4*)(yo + e));
  } else if (EB == 2) {
    uint16_t* yo = (uint16_t*)y + o;
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pk[e] = (uint32_t)f32_to_bf16(acc[2 * e]) | ((uint32_t)f32_to_bf16(acc[2 * e + 1]) << 16);
    __builtin_nontemporal_store(pk, (u32x4*)yo);
  } else {
    float* yo = (float*)y + o;
    __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, (f32x4*)yo);
  }
}

hipError_t launch_gather(const void* table, int64_t n_rows, int dim, int dtype, const int32_t* idx,
                         const float* w, int64_t n_bags, int bag, void* y, int y_dtype_is_table, hipStream_t s,
                         const void* z, int64_t z_ld, int z_bf16) {
  if (n_bags == 0) return hipSuccess;
  // one block per group of bags; a grid of at most 2^22 blocks (of <= 256 lanes: far below
  // the 2^32 work-items of one dispatch) loops over larger bag counts
  constexpr int64_t max_blocks = (int64_t)1 << 22;
  const int eb = dtype == DT_BF16 ? 2 : 4;
  const int row_vecs = (int)((int64_t)dim * eb / 16);
  if (z_ld == 0) z_ld = dim;
  const int tpr = row_vecs < 256 ? row_vecs : 256;
  const int bpb = 256 / tpr;
  const int threads = bpb * tpr;
  const int64_t groups = (n_bags + bpb - 1) / bpb;
  const int cols = (row_vecs + tpr - 1) / tpr;
  const int64_t bx = groups < max_blocks / cols ? groups : (max_blocks / cols > 0 ? max_blocks / cols : 1);
  dim3 grid((unsigned)bx, (unsigned)cols);
  const int y_f32 = (!y_dtype_is_table || dtype == DT_F32) ? 1 : 0;
  const bool uniform = (tpr % 64) == 0;
#define PKM_GATHER(EBV, UNI, ZBV)                                                                             \
  gather_kernel<EBV, 16, UNI, ZBV><<<grid, threads, 0, s>>>((const uint8_t*)table, n_rows, row_vecs, tpr, bpb, idx, \
                                                            w, n_bags, bag, y, y_f32, z, z_ld)
  // z rows whose start is not 16-byte aligned (a query width or head count that leaves the z
  // columns, or the row pitch, off a 16-byte multiple) take 4-byte loads
  const int zb = z_bf16 ? 2 : 4;
  const bool z16 = z && ((uintptr_t)z & 15) == 0 && (z_ld * zb) % 16 == 0;
  if (z && (((uintptr_t)z & 3) != 0 || (z_ld * zb) % 4 != 0)) return hipErrorInvalidValue;
  if (z && z_bf16) {
    if (eb != 2) return hipErrorInvalidValue;  // a bf16 z comes with bf16 values
    if (z16) {
      if (uniform) PKM_GATHER(2, true, 2); else PKM_GATHER(2, false, 2);
    } else {
      if (uniform) PKM_GATHER(2, true, -2); else PKM_GATHER(2, false, -2);
    }
  } else if (z) {
    if (eb == 2) {
      if (z16) {
        if (uniform) PKM_GATHER(2, true, 4); else PKM_GATHER(2, false, 4);
      } else {
        if (uniform) PKM_GATHER(2, true, -4); else PKM_GATHER(2, false, -4);
      }
    } else {
      if (z16) {
        if (uniform) PKM_GATHER(4, true, 4); else PKM_GATHER(4, false, 4);
      } else {
        if (uniform) PKM_GATHER(4, true, -4); else PKM_GATHER(4, false, -4);
      }
    }
  } else if (eb == 2) {
    if (uniform) PKM_GATHER(2, true, 0); else PKM_GATHER(2, false, 0);
  } else {
    if (uniform) PKM_GATHER(4, true, 0); else PKM_GATHER(4, false, 0);
  }
#undef PKM_GATHER
  return hipGetLastError();
}

}  // namespace pkm
