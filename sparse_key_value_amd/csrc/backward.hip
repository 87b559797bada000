// Backward of the weighted EmbeddingBag and the sparse update of the touched rows
// ("Memory Layers at Scale" digest, parallel EmbeddingBag: the forward sum whose chain
// rule this is; "Memory inside the model" overview, learning without forgetting: only
// the slots that were read are edited), and their C entry point.
//
//  * dw (and ds): one block of four waves per bag; each wave keeps the bag's dy row in
//    registers (dim <= 2048 floats: at most 32 per lane) and takes every fourth entry,
//    with four entries' table slices in flight per lane; a wave reduction gives each
//    dot product.  The table rows are read once, like the forward gather.
//  * the per-row sums: the (row, position) pairs are sorted by row with a stable radix
//    sort (rocPRIM device primitives).  Each touched row then has exactly one owner, the
//    first of its entries in position order, which sums w * dy over the row's positions
//    in position order (the result does not depend on scheduling, and no atomics are
//    used).
//  * the update runs per token, shaped like the forward gather: each lane keeps its
//    16-byte column slice of the token's dy in registers and walks the token's entries,
//    with several rows in flight; an entry that is its row's only one (most rows at
//    scale) is updated straight from those registers, an owner of a shared row walks
//    the row's sorted positions for the other tokens' dy, and the remaining entries
//    do nothing.  dy is thereby read about once, not once per entry.
//  * the gradient output, when asked for, comes from one block per distinct row (run
//    length encoding and a scan of the sorted keys give each row's output slot).
#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/device/device_run_length_encode.hpp>
#include <rocprim/device/device_scan.hpp>

#include <mutex>

#include "../../include/bag_backward.h"
#include "abi.hpp"
#include "checks.hpp"
#include "common.hpp"

namespace pkm {

namespace {

constexpr int MAX_BAG = BAG_MAX;

template <int EB>
struct BV;
template <>
struct BV<2> {
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
struct BV<4> {
  static constexpr int E = 4;
  __device__ static __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(v[e]);
  }
  __device__ static __forceinline__ u32x4 pack(const float* f) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
  }
};

// dy[b] slice s (E floats, 16-byte aligned).
template <int E>
__device__ __forceinline__ void load_dy(const float* p, float* d) {
#pragma unroll
  for (int x = 0; x < E; x += 4) {
    const f32x4 q = *(const f32x4*)(p + x);
    d[x] = q[0];
    d[x + 1] = q[1];
    d[x + 2] = q[2];
    d[x + 3] = q[3];
  }
}

// One block per bag.  SPL = 16-byte table slices per lane.
template <int EB, int SPL>
__global__ void __launch_bounds__(256) bag_dw_kernel(const uint8_t* __restrict__ table, int64_t n_rows, int slices,
                                                     int dim, const int32_t* __restrict__ idx,
                                                     const float* __restrict__ w, const float* __restrict__ dy,
                                                     int bag, float* __restrict__ dw, float* __restrict__ ds,
                                                     int group) {
  using V = BV<EB>;
  constexpr int E = V::E, U = 4;
  __shared__ float dws[MAX_BAG];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t b = blockIdx.x;

  float d[SPL][E];
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int s = lane + 64 * i;
    if (s < slices) {
      load_dy<E>(dy + b * dim + (int64_t)s * E, d[i]);
    } else {
#pragma unroll
      for (int x = 0; x < E; ++x) d[i][x] = 0.f;
    }
  }

  const int32_t* bi = idx + b * bag;
  const size_t row_bytes = (size_t)slices * 16;
  for (int j0 = wv; j0 < bag; j0 += 4 * U) {
    u32x4 v[U][SPL];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + 4 * u;
      const int32_t r = j < bag ? bi[j] : -1;
      ok[u] = r >= 0 && (int64_t)r < n_rows;
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int s = lane + 64 * i;
        v[u][i] = (ok[u] && s < slices)
                      ? __builtin_nontemporal_load((const u32x4*)(table + (size_t)r * row_bytes + (size_t)s * 16))
                      : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        float f[E];
        V::unpack(v[u][i], f);
#pragma unroll
        for (int x = 0; x < E; ++x) p = __builtin_fmaf(d[i][x], f[x], p);
      }
      p = wave_sum_f32(p);
      const int j = j0 + 4 * u;
      if (lane == 0 && j < bag) dws[j] = ok[u] ? p : 0.f;
    }
  }
  __syncthreads();
  for (int j = threadIdx.x; j < bag; j += 256) {
    const float g = dws[j];
    if (dw) dw[b * bag + j] = g;
    if (ds) {
      const int g0 = j - j % group;
      float sum = 0.f;
      for (int q = g0; q < g0 + group; ++q) sum = __builtin_fmaf(w[b * bag + q], dws[q], sum);
      ds[b * bag + j] = w[b * bag + j] * (g - sum);
    }
  }
}

// Sort keys: the row, or n_rows for an index that read nothing (those sort last).
__global__ void __launch_bounds__(256) bag_keys_kernel(const int32_t* __restrict__ idx, int64_t n, int64_t n_rows,
                                                       uint32_t* __restrict__ keys, uint32_t* __restrict__ vals) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int32_t r = idx[i];
  keys[i] = (r >= 0 && (int64_t)r < n_rows) ? (uint32_t)r : (uint32_t)n_rows;
  vals[i] = (uint32_t)i;
}

// One block per distinct row (grid-strided when the grid is smaller): the row's gradient
// in position order, into output slot u.  Also the distinct rows and their count.
template <int EB>
__global__ void __launch_bounds__(256) bag_grad_kernel(const uint32_t* __restrict__ unique,
                                                       const uint32_t* __restrict__ counts,
                                                       const uint32_t* __restrict__ offsets,
                                                       const uint32_t* __restrict__ runs,
                                                       const uint32_t* __restrict__ pos_sorted,
                                                       const float* __restrict__ w, const float* __restrict__ dy,
                                                       int bag, int dim, int slices, uint32_t n_rows,
                                                       int32_t* __restrict__ rows, float* __restrict__ grad,
                                                       int32_t* __restrict__ n_unique) {
  constexpr int E = BV<EB>::E;
  const uint32_t R = *runs;
  if (blockIdx.x == 0 && threadIdx.x == 0 && n_unique)
    n_unique[0] = (int32_t)((R > 0 && unique[R - 1] >= n_rows) ? R - 1 : R);
  for (uint32_t u = blockIdx.x; u < R; u += gridDim.x) {
    const uint32_t key = unique[u];
    if (key >= n_rows) continue;  // the run of indices that read nothing (always the last)
    const uint32_t off = offsets[u], cnt = counts[u];
    if (rows && threadIdx.x == 0) rows[u] = (int32_t)key;
    for (int s = threadIdx.x; s < slices; s += 256) {
      float acc[E];
#pragma unroll
      for (int x = 0; x < E; ++x) acc[x] = 0.f;
      for (uint32_t e = 0; e < cnt; ++e) {
        const uint32_t p = pos_sorted[off + e];
        const float wt = w[p];
        float dd[E];
        load_dy<E>(dy + (int64_t)(p / (uint32_t)bag) * dim + (int64_t)s * E, dd);
#pragma unroll
        for (int x = 0; x < E; ++x) acc[x] = __builtin_fmaf(wt, dd[x], acc[x]);
      }
      float* go = grad + (int64_t)u * dim + (int64_t)s * E;
#pragma unroll
      for (int x = 0; x < E; x += 4) *(f32x4*)(go + x) = f32x4{acc[x], acc[x + 1], acc[x + 2], acc[x + 3]};
    }
  }
}

// The distinct rows and their count, without gradients.
__global__ void __launch_bounds__(256) bag_rows_kernel(const uint32_t* __restrict__ unique,
                                                       const uint32_t* __restrict__ runs, int64_t n,
                                                       uint32_t n_rows, int32_t* __restrict__ rows,
                                                       int32_t* __restrict__ n_unique) {
  const uint32_t R = *runs;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u == 0 && n_unique) n_unique[0] = (int32_t)((R > 0 && unique[R - 1] >= n_rows) ? R - 1 : R);
  if (rows && u < (int64_t)R && u < n && unique[u] < n_rows) rows[u] = (int32_t)unique[u];
}

// The update role of every entry, from the row-sorted order (entry i of the order has
// key keys_sorted[i] and position pos_sorted[i]):
//   the row, when the entry is its row's only one;
//   -2 - i, when it is the first (in position order) of several entries of its row,
//     whose positions are pos_sorted[i], pos_sorted[i + 1], ... while the key stays;
//   -1 for the other entries of a shared row and for indices that read nothing.
// n < 2^31, so -2 - i fits an int32.  With dw, the entries that read nothing get dw = 0.
__global__ void __launch_bounds__(256) bag_owner_kernel(const uint32_t* __restrict__ keys_sorted,
                                                        const uint32_t* __restrict__ pos_sorted, int64_t n,
                                                        uint32_t n_rows, int32_t* __restrict__ role,
                                                        float* __restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const uint32_t key = keys_sorted[i];
  if (dw && key >= n_rows) dw[pos_sorted[i]] = 0.f;  // read nothing: dw = 0
  int32_t r;
  if (key >= n_rows || (i > 0 && keys_sorted[i - 1] == key)) r = -1;
  else if (i + 1 < n && keys_sorted[i + 1] == key) r = (int32_t)(-2 - i);
  else r = (int32_t)key;
  role[pos_sorted[i]] = r;
}

// table[row] slices -= lr * grad slices, rounded to the table's type; grad summed from
// zero with fp32 fmas in position order.  The rows are read with nontemporal loads and
// written with nontemporal stores: each touched row is read and written once, and with
// both hints the update runs about 10% faster on MI355X than with neither.
template <int EB, int SPL, int STRIDE>
__device__ __forceinline__ void apply_update(uint8_t* p, const bool* ok, const float (*acc)[BV<EB>::E], float lr,
                                             const u32x4* old) {
  using V = BV<EB>;
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    if (!ok[i]) continue;
    float t[V::E];
    V::unpack(old[i], t);
#pragma unroll
    for (int x = 0; x < V::E; ++x) t[x] = __builtin_fmaf(-lr, acc[i][x], t[x]);
    __builtin_nontemporal_store(V::pack(t), (u32x4*)(p + (size_t)i * STRIDE));
  }
}

// Sum over the token's lanes (WPG waves) of one value per lane, for UNROLL values at
// once; the totals are valid in lane 0 of the token's first wave.  WPG > 1: the block is
// one token, every wave calls this at the same point (`red` = two buffers of
// [4][UNROLL] floats used alternately, `buf` the one to use) and one barrier separates
// the writes from the reads.  Fixed order: a butterfly within each wave, then the waves
// in order.
template <int WPG, int UNROLL>
__device__ __forceinline__ void token_sum(float* v, float (*red)[4][UNROLL], int buf, int wig, int lane) {
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) v[u] = wave_sum_f32(v[u]);
  if constexpr (WPG > 1) {
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) red[buf][wig][u] = v[u];
    }
    __syncthreads();
    if (wig == 0) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        float t = red[buf][0][u];
#pragma unroll
        for (int q = 1; q < WPG; ++q) t += red[buf][q][u];
        v[u] = t;
      }
    }
  }
}

// One token per WPG waves (a block is one token when WPG > 1, four tokens, one per wave,
// when WPG == 1); lane t of a token owns the 16-byte column slices t, t + 64 * WPG, ...
// (SPL of them) of every row, and keeps the same slices of the token's dy in registers.
// The rows of the next UNROLL entries are loaded before the current ones are written, so
// that waiting for the loads does not wait for the stores (loads and stores share one
// counter).  An entry whose row is not updated from the registers loads row 0 instead
// (cached, discarded), so the loads need no branch.
// DW: also dw = <dy, old row> of every entry, from the rows the update reads anyway: a
// single-entry row's from the registers, a shared row's entries by the row's owner during
// its walk (before it writes the row), so no row is read twice.
template <int EB, int UNROLL, int SPL, int WPG, bool DW>
__global__ void __launch_bounds__(256) bag_update_kernel(uint8_t* __restrict__ table, int row_vecs,
                                                         const int32_t* __restrict__ role,
                                                         const uint32_t* __restrict__ keys_sorted,
                                                         const uint32_t* __restrict__ pos_sorted, int64_t n,
                                                         const float* __restrict__ w, const float* __restrict__ dy,
                                                         int64_t n_bags, int bag, float lr, float* __restrict__ dw) {
  using V = BV<EB>;
  constexpr int E = V::E;
  constexpr int TPB = WPG == 1 ? 4 : 1;  // tokens per block
  __shared__ float red[2][4][UNROLL];  // batch sums
  __shared__ float redw[2][4][1];      // sums during a shared row's walk
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wig = WPG == 1 ? 0 : wave;  // wave within the token
  const int64_t b = (int64_t)blockIdx.x * TPB + (WPG == 1 ? wave : 0);
  if (b >= n_bags) return;  // WPG > 1: the whole block, so no barrier is left waiting
  const int t = wig * 64 + lane;
  const int64_t dim = (int64_t)row_vecs * E;
  const size_t row_bytes = (size_t)row_vecs * 16;
  uint8_t* base = table + (size_t)t * 16;
  bool ok[SPL];
  float d[SPL][E];
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    ok[i] = t + i * 64 * WPG < row_vecs;
    if (ok[i]) {
      load_dy<E>(dy + b * dim + (int64_t)(t + i * 64 * WPG) * E, d[i]);
    } else {
#pragma unroll
      for (int x = 0; x < E; ++x) d[i][x] = 0.f;
    }
  }
  const int32_t* br = role + b * bag;
  const float* bw = w + b * bag;
  int buf = 0, wbuf = 0;
  auto fetch = [&](int j, int32_t* r, u32x4 (*v)[SPL]) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      r[u] = j + u < bag ? br[j + u] : -1;
      const uint8_t* rp = base + (size_t)(r[u] >= 0 ? r[u] : 0) * row_bytes;
#pragma unroll
      for (int i = 0; i < SPL; ++i)
        v[u][i] = ok[i] ? __builtin_nontemporal_load((const u32x4*)(rp + (size_t)i * (64 * WPG * 16)))
                        : u32x4{0u, 0u, 0u, 0u};
    }
  };
  int32_t r[UNROLL];
  u32x4 v[UNROLL][SPL];
  fetch(0, r, v);
  for (int j = 0; j < bag; j += UNROLL) {
    int32_t rn[UNROLL];
    u32x4 vn[UNROLL][SPL];
    fetch(j + UNROLL, rn, vn);
    if constexpr (DW) {
      // dw of the single-entry rows of this batch, from the old rows in registers
      float pd[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        pd[u] = 0.f;
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
          float f[E];
          V::unpack(v[u][i], f);
#pragma unroll
          for (int x = 0; x < E; ++x) pd[u] = __builtin_fmaf(d[i][x], f[x], pd[u]);
        }
      }
      token_sum<WPG, UNROLL>(pd, red, buf, wig, lane);
      buf ^= 1;
      if (wig == 0 && lane == 0) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
          if (r[u] >= 0) dw[b * bag + j + u] = pd[u];
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if (r[u] >= 0) {
        float acc[SPL][E];
#pragma unroll
        for (int i = 0; i < SPL; ++i)
#pragma unroll
          for (int x = 0; x < E; ++x) acc[i][x] = __builtin_fmaf(bw[j + u], d[i][x], 0.f);
        apply_update<EB, SPL, 64 * WPG * 16>(base + (size_t)r[u] * row_bytes, ok, acc, lr, v[u]);
      } else if (r[u] <= -2) {
        // the owner of a shared row: its entries' gradient sum (and dw) in position order
        const int64_t i0 = -2 - (int64_t)r[u];
        const uint32_t key = keys_sorted[i0];
        uint8_t* tp = base + (size_t)key * row_bytes;
        u32x4 old[SPL];
#pragma unroll
        for (int i = 0; i < SPL; ++i)
          old[i] = ok[i] ? __builtin_nontemporal_load((const u32x4*)(tp + (size_t)i * (64 * WPG * 16)))
                         : u32x4{0u, 0u, 0u, 0u};
        float acc[SPL][E];
#pragma unroll
        for (int i = 0; i < SPL; ++i)
#pragma unroll
          for (int x = 0; x < E; ++x) acc[i][x] = 0.f;
        for (int64_t q = i0; q < n && keys_sorted[q] == key; ++q) {
          const uint32_t p = pos_sorted[q];
          const float wt = w[p];
          const float* dyp = dy + (int64_t)(p / (uint32_t)bag) * dim + (int64_t)t * E;
          float pd[1] = {0.f};
#pragma unroll
          for (int i = 0; i < SPL; ++i) {
            if (!ok[i]) continue;
            float dd[E];
            load_dy<E>(dyp + (int64_t)i * 64 * WPG * E, dd);
#pragma unroll
            for (int x = 0; x < E; ++x) acc[i][x] = __builtin_fmaf(wt, dd[x], acc[i][x]);
            if constexpr (DW) {
              float f[E];
              V::unpack(old[i], f);
#pragma unroll
              for (int x = 0; x < E; ++x) pd[0] = __builtin_fmaf(dd[x], f[x], pd[0]);
            }
          }
          if constexpr (DW) {
            token_sum<WPG, 1>(pd, redw, wbuf, wig, lane);
            wbuf ^= 1;
            if (wig == 0 && lane == 0) dw[p] = pd[0];
          }
        }
        apply_update<EB, SPL, 64 * WPG * 16>(tp, ok, acc, lr, old);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      r[u] = rn[u];
#pragma unroll
      for (int i = 0; i < SPL; ++i) v[u][i] = vn[u][i];
    }
  }
}

// ds from dw: ds[i] = w[i] * (dw[i] - sum over i's softmax group of w * dw), the sum in
// position order.
__global__ void __launch_bounds__(256) bag_ds_kernel(const float* __restrict__ w, const float* __restrict__ dw,
                                                     int64_t n, int group, float* __restrict__ ds) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t g0 = i - i % group;
  float sum = 0.f;
  for (int64_t q = g0; q < g0 + group; ++q) sum = __builtin_fmaf(w[q], dw[q], sum);
  ds[i] = w[i] * (dw[i] - sum);
}

struct SortSpace {
  size_t keys = 0, keys_sorted = 0, vals = 0, vals_sorted = 0, unique = 0, counts = 0, offsets = 0, runs = 0,
         temp = 0, temp_bytes = 0, total = 0;
};

unsigned key_bits(int64_t n_rows) {
  unsigned b = 1;
  while (b < 32 && ((uint64_t)1 << b) <= (uint64_t)n_rows) ++b;  // n_rows itself (the sentinel) must fit
  return b;
}

// Buffers of the sort and their rocPRIM temporary storage (sizes from rocPRIM's own queries).
int sort_space(int64_t n, int64_t n_rows, SortSpace& S) {
  auto a = [](size_t v) { return (v + 255) & ~(size_t)255; };
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = a(off + bytes);
    return o;
  };
  S.keys = take(n * 4);
  S.keys_sorted = take(n * 4);
  S.vals = take(n * 4);
  S.vals_sorted = take(n * 4);
  S.unique = take(n * 4);
  S.counts = take(n * 4);
  S.offsets = take(n * 4);
  S.runs = take(4);
  size_t t1 = 0, t2 = 0, t3 = 0;
  const unsigned bits = key_bits(n_rows);
  PKM_HIP(rocprim::radix_sort_pairs(nullptr, t1, (const uint32_t*)nullptr, (uint32_t*)nullptr,
                                    (const uint32_t*)nullptr, (uint32_t*)nullptr, (uint32_t)n, 0u, bits));
  PKM_HIP(rocprim::run_length_encode(nullptr, t2, (const uint32_t*)nullptr, (unsigned)n, (uint32_t*)nullptr,
                                     (uint32_t*)nullptr, (uint32_t*)nullptr));
  PKM_HIP(rocprim::exclusive_scan(nullptr, t3, (const uint32_t*)nullptr, (uint32_t*)nullptr, 0u, (size_t)n,
                                  rocprim::plus<uint32_t>()));
  S.temp_bytes = t1 > t2 ? (t1 > t3 ? t1 : t3) : (t2 > t3 ? t2 : t3);
  S.temp = take(S.temp_bytes);
  S.total = off;
  return PKM_OK;
}

int check_sizes(int64_t n_bags, int32_t bag_size, int64_t n_rows) {
  const std::string why = check_bag_sizes(n_bags, bag_size, n_rows);
  return why.empty() ? PKM_OK : pkm_abi::fail(PKM_EINVAL, "%s", why.c_str());
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

template <int EB>
int launch_dw(const pkm_bag_backward_args* a, const uint8_t* table, int slices, hipStream_t s) {
  const int spl = (slices + 63) / 64;
  const dim3 grid((unsigned)a->n_bags);
#define PKM_DW(SPLV)                                                                                            \
  PKM_LAUNCH((bag_dw_kernel<EB, SPLV><<<grid, 256, 0, s>>>(table, a->n_rows, slices, a->dim, a->idx, a->w, a->dy, \
                                                           a->bag_size, a->dw, a->ds, a->softmax_group),         \
              hipGetLastError()))
  if (spl == 1) PKM_DW(1);
  else if (spl == 2) PKM_DW(2);
  else if (spl <= 4) PKM_DW(4);
  else PKM_DW(8);
#undef PKM_DW
  return PKM_OK;
}

// One token per 1, 2 or 4 waves (the fewest that give every lane at most two slices);
// eight rows in flight per lane.
template <int EB>
int launch_update(const pkm_bag_backward_args* a, uint8_t* table, int slices, const int32_t* role,
                  const uint32_t* keys_sorted, const uint32_t* pos_sorted, float* dw, hipStream_t s) {
  const int wpg = slices <= 64 ? 1 : (slices <= 128 ? 2 : 4);
  const int spl = (slices + 64 * wpg - 1) / (64 * wpg);
  const int tpb = wpg == 1 ? 4 : 1;
  const dim3 grid((unsigned)((a->n_bags + tpb - 1) / tpb));
  const int threads = wpg == 1 ? 256 : 64 * wpg;
  const int64_t n = a->n_bags * a->bag_size;
#define PKM_UPD(SPLV, WPGV, DWV)                                                                             \
  PKM_LAUNCH((bag_update_kernel<EB, 8 / SPLV, SPLV, WPGV, DWV><<<grid, threads, 0, s>>>(                       \
                  table, slices, role, keys_sorted, pos_sorted, n, a->w, a->dy, a->n_bags, a->bag_size, a->lr, \
                  dw),                                                                                       \
              hipGetLastError()))
#define PKM_UPD_DW(SPLV, WPGV) \
  do {                         \
    if (dw) PKM_UPD(SPLV, WPGV, true); \
    else PKM_UPD(SPLV, WPGV, false);   \
  } while (0)
  if (wpg == 1) PKM_UPD_DW(1, 1);
  else if (wpg == 2) PKM_UPD_DW(1, 2);
  else if (spl == 1) PKM_UPD_DW(1, 4);
  else PKM_UPD_DW(2, 4);
#undef PKM_UPD_DW
#undef PKM_UPD
  return PKM_OK;
}

// Sort buffers for callers that cannot allocate device memory (pkm_bag_backward_noalloc):
// a fixed array that every GPU the library runs on holds until the process ends.  In host
// code the name `scratch` stands for the array but is not its device address: kernels and
// copies are given the address hipGetSymbolAddress returns for the current device, which
// is looked up once per device and kept.  Every call on one GPU shares that GPU's array.
// Nothing in it has to start at zero: the kernels and the rocPRIM primitives write every
// byte of it they later read.
static __device__ __align__(256) uint8_t scratch[PKM_BAG_BACKWARD_NOALLOC_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The current device's address of `scratch` (looked up on the device's first call).
int scratch_address(void** out) {
  using pkm_abi::fail;
  int dev = 0;
  PKM_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(PKM_EUNSUPPORTED, "device index %d is not below %d", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PKM_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKM_OK;
}

// The backward on `s`.  The sort buffers are the caller's workspace (ws, ws_bytes), or, with
// `fixed`, the library's scratch array of ws_bytes on the current device.  Every argument and
// size is checked before anything is enqueued.
int run_bag_backward(const pkm_bag_backward_args* a, uint8_t* ws, size_t ws_bytes, bool fixed, hipStream_t s) {
  using pkm_abi::fail;
  if (!a) return fail(PKM_EINVAL, "args is NULL");
  int rc = check_sizes(a->n_bags, a->bag_size, a->n_rows);
  if (rc != PKM_OK) return rc;
  if (a->dtype != PKM_F32 && a->dtype != PKM_BF16) return fail(PKM_EINVAL, "dtype must be PKM_F32 or PKM_BF16");
  const int eb = a->dtype == PKM_BF16 ? 2 : 4;
  if (a->dim < 1 || a->dim > 2048 || ((int64_t)a->dim * eb) % 16 != 0)
    return fail(PKM_EINVAL, "dim must be in [1, 2048] with dim * sizeof(dtype) a multiple of 16");
  if (a->ds && (a->softmax_group < 1 || a->bag_size % a->softmax_group != 0))
    return fail(PKM_EINVAL, "softmax_group must divide bag_size");
  if (a->update != 0 && a->update != 1) return fail(PKM_EINVAL, "update must be 0 or 1");
  if (a->n_bags == 0) return PKM_OK;
  if (!a->table || !a->idx || !a->w || !a->dy) return fail(PKM_EINVAL, "table, idx, w and dy must not be NULL");
  if ((((uintptr_t)a->table | (uintptr_t)a->dy | (uintptr_t)a->grad) & 15) != 0)
    return fail(PKM_EINVAL, "table, dy and grad must be 16-byte aligned");
  const bool need_sort = a->rows || a->grad || a->n_unique || a->update;
  if ((rc = device_ok()) != PKM_OK) return rc;
  const void* tview = nullptr;
  if ((rc = pkm_abi::device_view(a->table, "table", &tview)) != PKM_OK) return rc;
  const int slices = a->dim * eb / 16;
  const int64_t n = a->n_bags * a->bag_size;
  SortSpace S;
  if (need_sort) {
    if ((rc = sort_space(n, a->n_rows, S)) != PKM_OK) return rc;
    if (fixed) {
      if (S.total > ws_bytes)
        return fail(PKM_EWORKSPACE, "these sizes need %zu bytes of sort buffers, more than the library's fixed %zu "
                    "(pkm_bag_backward with a workspace takes any size)", S.total, ws_bytes);
      void* p = nullptr;
      if ((rc = scratch_address(&p)) != PKM_OK) return rc;
      ws = (uint8_t*)p;
    } else {
      if (!ws || ws_bytes < S.total)
        return fail(PKM_EWORKSPACE, "workspace has %zu bytes, these sizes need %zu", ws ? ws_bytes : (size_t)0,
                    S.total);
      if (((uintptr_t)ws & 255) != 0) return fail(PKM_EINVAL, "workspace must be 256-byte aligned");
      if ((rc = pkm_abi::require_device(ws, "workspace")) != PKM_OK) return rc;
    }
  }

  // without the update, dw and ds come from their own pass over the rows; with it, from
  // the rows the update reads (before writing them)
  if ((a->dw || a->ds) && !a->update) {
    if (a->dtype == PKM_BF16) rc = launch_dw<2>(a, (const uint8_t*)tview, slices, s);
    else rc = launch_dw<4>(a, (const uint8_t*)tview, slices, s);
    if (rc != PKM_OK) return rc;
  }
  if (!need_sort) return PKM_OK;
  auto U = [&](size_t o) { return (uint32_t*)(ws + o); };
  PKM_LAUNCH((bag_keys_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(a->idx, n, a->n_rows,
                                                                                   U(S.keys), U(S.vals)),
              hipGetLastError()));
  size_t tb = S.temp_bytes;
  PKM_HIP(rocprim::radix_sort_pairs(ws + S.temp, tb, (const uint32_t*)U(S.keys), U(S.keys_sorted),
                                    (const uint32_t*)U(S.vals), U(S.vals_sorted), (uint32_t)n, 0u,
                                    key_bits(a->n_rows), s));
  if (a->update) {
    // roles into the unsorted-key buffer and, when only ds is asked for, dw into the
    // unsorted-position buffer: the sort has finished with both
    int32_t* role = (int32_t*)U(S.keys);
    float* dwp = a->dw ? a->dw : (a->ds ? (float*)U(S.vals) : nullptr);
    const uint32_t* ks = U(S.keys_sorted);
    const uint32_t* ps = U(S.vals_sorted);
    PKM_LAUNCH((bag_owner_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(ks, ps, n, (uint32_t)a->n_rows,
                                                                                      role, dwp),
                hipGetLastError()));
    if (a->dtype == PKM_BF16) rc = launch_update<2>(a, (uint8_t*)tview, slices, role, ks, ps, dwp, s);
    else rc = launch_update<4>(a, (uint8_t*)tview, slices, role, ks, ps, dwp, s);
    if (rc != PKM_OK) return rc;
    if (a->ds)
      PKM_LAUNCH((bag_ds_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(a->w, dwp, n, a->softmax_group,
                                                                                     a->ds),
                  hipGetLastError()));
  }
  if (!a->rows && !a->grad && !a->n_unique) return PKM_OK;
  tb = S.temp_bytes;
  PKM_HIP(rocprim::run_length_encode(ws + S.temp, tb, (const uint32_t*)U(S.keys_sorted), (unsigned)n, U(S.unique),
                                     U(S.counts), U(S.runs), s));
  if (!a->grad) {
    PKM_LAUNCH((bag_rows_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(
                   U(S.unique), U(S.runs), n, (uint32_t)a->n_rows, a->rows, a->n_unique),
                hipGetLastError()));
    return PKM_OK;
  }
  tb = S.temp_bytes;
  PKM_HIP(rocprim::exclusive_scan(ws + S.temp, tb, (const uint32_t*)U(S.counts), U(S.offsets), 0u, (size_t)n,
                                  rocprim::plus<uint32_t>(), s));
  // one block per possible run (at most n, the grid capped at 2^22 blocks, which then loop): a
  // block's rows form a chain of dependent loads, so many resident blocks are what hides the
  // latency; blocks past the run count exit
  const dim3 grid((unsigned)(n < ((int64_t)1 << 22) ? n : ((int64_t)1 << 22)));
#define PKM_GRAD(EBV)                                                                                          \
  PKM_LAUNCH((bag_grad_kernel<EBV><<<grid, 256, 0, s>>>(U(S.unique), U(S.counts), U(S.offsets), U(S.runs), \
                                                             U(S.vals_sorted), a->w, a->dy, a->bag_size, a->dim, \
                                                             slices, (uint32_t)a->n_rows, a->rows, a->grad,      \
                                                             a->n_unique),                                       \
              hipGetLastError()))
  if (a->dtype == PKM_BF16) PKM_GRAD(2);
  else PKM_GRAD(4);
#undef PKM_GRAD
  return PKM_OK;
}


}  // namespace

}  // namespace pkm

extern "C" {

size_t pkm_bag_backward_workspace_size(int64_t n_bags, int32_t bag_size, int64_t n_rows) {
  if (pkm::check_sizes(n_bags, bag_size, n_rows) != PKM_OK) return 0;
  pkm::SortSpace S;
  if (pkm::sort_space(n_bags * bag_size > 0 ? n_bags * bag_size : 1, n_rows, S) != PKM_OK) return 0;
  return S.total;
}

int pkm_bag_backward(const pkm_bag_backward_args* a, void* workspace, size_t ws_bytes, void* stream) {
  return pkm::run_bag_backward(a, (uint8_t*)workspace, ws_bytes, false, (hipStream_t)stream);
}

int pkm_bag_backward_noalloc(const pkm_bag_backward_args* a, void* stream) {
  return pkm::run_bag_backward(a, nullptr, PKM_BAG_BACKWARD_NOALLOC_BYTES, true, (hipStream_t)stream);
}

}  // extern "C"
