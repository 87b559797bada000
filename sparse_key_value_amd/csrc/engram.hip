// Hashed n-gram lookup (review of "Conditional Memory via Scalable Lookup" (Engram):
// sparse retrieval with multi-head hashing, key equation 1; context-aware gating, key
// equation 2; residual connection) and its C entry points.
//
// One wave per token does the whole lookup: the token ids of the longest n-gram ending
// at the token are read once (wave-uniform); lane p folds the hash of (order, head)
// pair p (one hash per lane instead of one per lane and slice) and leaves the row in
// LDS; every lane then puts all the rows of its 16-byte column slices in flight at once
// (nontemporal: the tables are far larger than the caches), sums the orders in fp32,
// and the wave reduces <h, e>, |h|^2 and |e|^2 for the gate before writing
// alpha * e (+ h).  The modulus uses an fp64 reciprocal of P and an exact integer
// correction instead of a 64-bit division.  The embedding is never written to memory unless asked for,
// so a token costs its table rows, its hidden state and its output: for 2 orders x 8
// heads x 128 bf16 at d = 1024, 4 KiB + 2 KiB + 2 KiB.
#include <string>

#include "../../include/engram.h"
#include "abi.hpp"
#include "checks.hpp"
#include "common.hpp"

namespace pkm {

namespace {

constexpr int MAX_ORDER = ENGRAM_MAX_ORDER;
constexpr int MAX_ORDERS = ENGRAM_MAX_ORDERS;

struct EngramArgs {
  const uint8_t* tables;
  const int32_t* ids;
  const int32_t* compress;
  const uint64_t* mult;
  const uint8_t* h;
  uint8_t* out;
  float* e_out;
  float* alpha_out;
  int64_t T, seq_len, P;
  int vocab, min_order, n_orders, heads;
  int head_vecs;  // 16-byte slices of one table row
  int slices;     // 16-byte slices of a token's d values
  int d, residual;
  float eps;
  double inv_p;      // 1 / P, rounded
  uint64_t two32_p;  // 2^32 mod P
  uint8_t* staged;   // [T, n_orders, d] rows copied ahead of use (prefetch / staged modes)
};

// What one launch of the token kernel does.
enum Mode {
  FULL = 0,      // hash, read the table rows, gate, write the output
  PREFETCH = 1,  // hash, read the table rows (e.g. from host memory), write them to `staged`
  STAGED = 2,    // read the rows from `staged`, gate, write the output
};

// The id the hash sees (ids outside [0, vocab) read as 0; optional vocabulary map).
__device__ __forceinline__ uint64_t norm_id(const EngramArgs& a, int64_t j) {
  int32_t v = a.ids[j];
  v = (v >= 0 && v < a.vocab) ? v : 0;
  return a.compress ? (uint64_t)(uint32_t)a.compress[v] : (uint64_t)(uint32_t)v;
}

// phi before the modulus: fold of the last n of the MAX_ORDER ids in `tok` (oldest first).
__device__ __forceinline__ uint64_t fold(const uint64_t (&tok)[MAX_ORDER], int n, uint64_t m) {
  uint64_t hh = 0;
#pragma unroll
  for (int i = 0; i < MAX_ORDER; ++i)
    if (i >= MAX_ORDER - n) hh = (hh ^ tok[i]) * m;
  return hh;
}

// x mod P for x / P < 2^40: the fp64 quotient estimate is off by at most one, which the
// two compares correct exactly.
__device__ __forceinline__ uint64_t mod_small(uint64_t x, uint64_t P, double inv_p) {
  const uint64_t q = (uint64_t)((double)x * inv_p);
  int64_t r = (int64_t)(x - q * P);
  r = r < 0 ? r + (int64_t)P : r;
  r = r >= (int64_t)P ? r - (int64_t)P : r;
  return (uint64_t)r;
}

// h mod P for any 64-bit h and 1 <= P < 2^31: h = hi * 2^32 + lo, so
// h mod P = ((hi mod P) * (2^32 mod P) + lo) mod P, whose operand is < 2^62 + 2^32 and
// whose quotient is < 2^32 + 2^32 / P.
__device__ __forceinline__ uint64_t mod_p(uint64_t h, const EngramArgs& a) {
  const uint64_t P = (uint64_t)a.P;
  const uint64_t r1 = mod_small(h >> 32, P, a.inv_p);
  return mod_small(r1 * a.two32_p + (h & 0xFFFFFFFFull), P, a.inv_p);
}

template <int EB>
struct Elems;
template <>
struct Elems<2> {
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
struct Elems<4> {
  static constexpr int E = 4;
  __device__ static __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(v[e]);
  }
  __device__ static __forceinline__ u32x4 pack(const float* f) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
  }
};

// Four tokens per block, one per wave; SPL = 16-byte slices of a token per lane.
template <int EB, int SPL, int MODE>
__global__ void __launch_bounds__(256) engram_forward_kernel(EngramArgs a) {
  using EL = Elems<EB>;
  constexpr int E = EL::E;
  __shared__ int32_t rows_s[4][MAX_ORDERS * 64];
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = (int64_t)blockIdx.x * 4 + wv;
  if (t >= a.T) return;

  // slices of this lane and its hidden-state values (independent of the hashes)
  u32x4 hv[SPL];
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int s = lane + 64 * i;
    hv[i] = (MODE != PREFETCH && s < a.slices) ? *(const u32x4*)(a.h + ((size_t)t * a.slices + s) * 16)
                                               : u32x4{0u, 0u, 0u, 0u};
  }

  u32x4 v[MAX_ORDERS][SPL];
  if constexpr (MODE == STAGED) {
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int s = lane + 64 * i;
#pragma unroll
      for (int o = 0; o < MAX_ORDERS; ++o)
        v[o][i] = (s < a.slices && o < a.n_orders)
                      ? __builtin_nontemporal_load((const u32x4*)(a.staged + (((size_t)t * a.n_orders + o) * a.slices + s) * 16))
                      : u32x4{0u, 0u, 0u, 0u};
    }
  } else {
  // ids of the longest n-gram ending at t, oldest first; before the sequence start: 0
  const int nmax = a.min_order + a.n_orders - 1;
  const int64_t start = t - t % a.seq_len;
  uint64_t tok[MAX_ORDER];
#pragma unroll
  for (int i = 0; i < MAX_ORDER; ++i) {
    const int64_t j = t - (MAX_ORDER - 1 - i);
    tok[i] = (i >= MAX_ORDER - nmax && j >= start) ? norm_id(a, j) : 0ull;
  }

  // lane p hashes (order, head) pair p = o * heads + k into the row of the stacked table
  const int pairs = a.n_orders * a.heads;
  for (int p = lane; p < pairs; p += 64) {
    const int o = p / a.heads;
    const uint64_t phi = mod_p(fold(tok, a.min_order + o, a.mult[p]), a);
    rows_s[wv][p] = (int32_t)((int64_t)p * a.P + (int64_t)phi);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // every row of this lane's slices in flight at once
  const size_t row_bytes = (size_t)a.head_vecs * 16;
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int s = lane + 64 * i;
    const bool ok = s < a.slices;
    const int k = ok ? s / a.head_vecs : 0;
    const int col = ok ? s - k * a.head_vecs : 0;
#pragma unroll
    for (int o = 0; o < MAX_ORDERS; ++o) {
      v[o][i] = u32x4{0u, 0u, 0u, 0u};
      if (ok && o < a.n_orders) {
        const int64_t row = rows_s[wv][o * a.heads + k];
        v[o][i] = __builtin_nontemporal_load((const u32x4*)(a.tables + (size_t)row * row_bytes + (size_t)col * 16));
      }
    }
  }
  if constexpr (MODE == PREFETCH) {
    // the rows of order o, head k land where the staged mode reads them: [t, o, slice]
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int s = lane + 64 * i;
#pragma unroll
      for (int o = 0; o < MAX_ORDERS; ++o)
        if (s < a.slices && o < a.n_orders)
          __builtin_nontemporal_store(v[o][i], (u32x4*)(a.staged + (((size_t)t * a.n_orders + o) * a.slices + s) * 16));
    }
    return;
  }
  }

  // e = sum over orders (fp32, order 0 first); the three sums of the gate
  float e[SPL][E], hf[SPL][E];
  float ee = 0.f, hh = 0.f, eh = 0.f;
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
#pragma unroll
    for (int x = 0; x < E; ++x) e[i][x] = 0.f;
#pragma unroll
    for (int o = 0; o < MAX_ORDERS; ++o) {
      float f[E];
      EL::unpack(v[o][i], f);
#pragma unroll
      for (int x = 0; x < E; ++x) e[i][x] += f[x];
    }
    EL::unpack(hv[i], hf[i]);
#pragma unroll
    for (int x = 0; x < E; ++x) {
      ee = __builtin_fmaf(e[i][x], e[i][x], ee);
      hh = __builtin_fmaf(hf[i][x], hf[i][x], hh);
      eh = __builtin_fmaf(hf[i][x], e[i][x], eh);
    }
  }
  ee = wave_sum_f32(ee);
  hh = wave_sum_f32(hh);
  eh = wave_sum_f32(eh);
  const float inv_d = 1.0f / (float)a.d;
  const float z = eh / (__fsqrt_rn(hh * inv_d + a.eps) * __fsqrt_rn(ee * inv_d + a.eps) * __fsqrt_rn((float)a.d));
  const float alpha = 1.0f / (1.0f + __expf(-z));

#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int s = lane + 64 * i;
    if (s >= a.slices) continue;
    float o[E];
#pragma unroll
    for (int x = 0; x < E; ++x) o[x] = a.residual ? __builtin_fmaf(alpha, e[i][x], hf[i][x]) : alpha * e[i][x];
    __builtin_nontemporal_store(EL::pack(o), (u32x4*)(a.out + ((size_t)t * a.slices + s) * 16));
    if (a.e_out) {
      float* eo = a.e_out + (size_t)t * a.d + (size_t)s * E;
#pragma unroll
      for (int x = 0; x < E; x += 4) *(f32x4*)(eo + x) = f32x4{e[i][x], e[i][x + 1], e[i][x + 2], e[i][x + 3]};
    }
  }
  if (a.alpha_out && lane == 0) a.alpha_out[t] = alpha;
}

// rows[i] of the hash, i = (t * heads + k) * n_orders + o.
__device__ __forceinline__ void hash_one(const EngramArgs& a, int32_t* __restrict__ rows, int64_t i) {
  const int o = (int)(i % a.n_orders);
  const int k = (int)((i / a.n_orders) % a.heads);
  const int64_t t = i / ((int64_t)a.n_orders * a.heads);
  const int n = a.min_order + o;
  const int64_t start = t - t % a.seq_len;
  const uint64_t m = a.mult[o * a.heads + k];
  uint64_t hh = 0;
  for (int64_t j = t - n + 1; j <= t; ++j) hh = (hh ^ (j >= start ? norm_id(a, j) : 0ull)) * m;
  rows[i] = (int32_t)(((int64_t)o * a.heads + k) * a.P + (int64_t)mod_p(hh, a));
}

// One thread per (token, head, order): rows[t, k, o]; a capped grid loops.
__global__ void __launch_bounds__(256) engram_hash_kernel(EngramArgs a, int32_t* __restrict__ rows) {
  const int64_t total = a.T * a.heads * a.n_orders;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256)
    hash_one(a, rows, i);
}

// Argument checks shared by both entry points; fills `a` on success.
int prepare(const engram_config* cfg, const int32_t* ids, int64_t T, int64_t seq_len, const int32_t* compress,
            const uint64_t* mult, EngramArgs& a) {
  std::string why = check_engram(cfg);
  if (!why.empty()) return pkm_abi::fail(PKM_EINVAL, "invalid engram config: %s", why.c_str());
  why = check_engram_tokens(T, seq_len);
  if (!why.empty()) return pkm_abi::fail(PKM_EINVAL, "%s", why.c_str());
  if (T > 0 && (!ids || !mult)) return pkm_abi::fail(PKM_EINVAL, "ids and mult must not be NULL");
  const int eb = cfg->dtype == PKM_BF16 ? 2 : 4;
  a = EngramArgs{};
  a.ids = ids;
  a.compress = compress;
  a.mult = mult;
  a.T = T;
  a.seq_len = seq_len;
  a.P = cfg->table_rows;
  a.vocab = cfg->vocab;
  a.min_order = cfg->min_order;
  a.n_orders = cfg->n_orders;
  a.heads = cfg->n_heads;
  a.head_vecs = cfg->head_dim * eb / 16;
  a.slices = a.heads * a.head_vecs;
  a.d = cfg->n_heads * cfg->head_dim;
  a.residual = cfg->residual;
  a.eps = cfg->norm_eps;
  a.inv_p = 1.0 / (double)cfg->table_rows;
  a.two32_p = ((uint64_t)1 << 32) % (uint64_t)cfg->table_rows;
  return PKM_OK;
}

// One launch of the token kernel: four tokens per block, instantiated per element size,
// slices per lane (1, 2 or 4) and mode.
template <int MODE>
int launch_mode(int dtype, const EngramArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.T + 3) / 4));
  const int spl = (a.slices + 63) / 64;  // 1..4
#define PKM_ENGRAM(EBV, SPLV) \
  PKM_LAUNCH((engram_forward_kernel<EBV, SPLV, MODE><<<grid, 256, 0, s>>>(a), hipGetLastError()))
  if (dtype == PKM_BF16) {
    if (spl == 1) PKM_ENGRAM(2, 1); else if (spl == 2) PKM_ENGRAM(2, 2); else PKM_ENGRAM(2, 4);
  } else {
    if (spl == 1) PKM_ENGRAM(4, 1); else if (spl == 2) PKM_ENGRAM(4, 2); else PKM_ENGRAM(4, 4);
  }
#undef PKM_ENGRAM
  return PKM_OK;
}

int launch_tokens(int dtype, int mode, const EngramArgs& a, hipStream_t s) {
  if (mode == PREFETCH) return launch_mode<PREFETCH>(dtype, a, s);
  if (mode == STAGED) return launch_mode<STAGED>(dtype, a, s);
  return launch_mode<FULL>(dtype, a, s);
}

// The device check once per device and process.
int device_ok() {
  static int state[64] = {};  // 0 unknown, 1 gfx950
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

int engram_hash(const engram_config* cfg, const int32_t* ids, int64_t T, int64_t seq_len, const int32_t* compress,
                const uint64_t* mult, int32_t* rows, void* stream) {
  pkm::EngramArgs a;
  int rc = pkm::prepare(cfg, ids, T, seq_len, compress, mult, a);
  if (rc != PKM_OK) return rc;
  if (T == 0) return PKM_OK;
  if (!rows) return pkm_abi::fail(PKM_EINVAL, "rows must not be NULL");
  if ((rc = pkm::device_ok()) != PKM_OK) return rc;
  const int64_t total = T * a.heads * a.n_orders;
  const int64_t blocks = (total + 255) / 256 < ((int64_t)1 << 20) ? (total + 255) / 256 : ((int64_t)1 << 20);
  PKM_LAUNCH((pkm::engram_hash_kernel<<<dim3((unsigned)blocks), 256, 0, (hipStream_t)stream>>>(a, rows),
              hipGetLastError()));
  return PKM_OK;
}

int engram_forward(const engram_config* cfg, const void* tables, const int32_t* ids, int64_t T, int64_t seq_len,
                   const int32_t* compress, const uint64_t* mult, const void* h, void* out, float* e_out,
                   float* alpha_out, void* stream) {
  pkm::EngramArgs a;
  int rc = pkm::prepare(cfg, ids, T, seq_len, compress, mult, a);
  if (rc != PKM_OK) return rc;
  if (T == 0) return PKM_OK;
  if (!tables || !h || !out) return pkm_abi::fail(PKM_EINVAL, "tables, h and out must not be NULL");
  if ((((uintptr_t)tables | (uintptr_t)h | (uintptr_t)out | (uintptr_t)e_out) & 15) != 0)
    return pkm_abi::fail(PKM_EINVAL, "tables, h, out and e_out must be 16-byte aligned");
  if ((rc = pkm::device_ok()) != PKM_OK) return rc;
  a.tables = (const uint8_t*)tables;
  a.h = (const uint8_t*)h;
  a.out = (uint8_t*)out;
  a.e_out = e_out;
  a.alpha_out = alpha_out;
  return pkm::launch_tokens(cfg->dtype, pkm::FULL, a, (hipStream_t)stream);
}

int engram_prefetch(const engram_config* cfg, const void* tables, const int32_t* ids, int64_t T, int64_t seq_len,
                    const int32_t* compress, const uint64_t* mult, void* staged, void* stream) {
  pkm::EngramArgs a;
  int rc = pkm::prepare(cfg, ids, T, seq_len, compress, mult, a);
  if (rc != PKM_OK) return rc;
  if (T == 0) return PKM_OK;
  if (!tables || !staged) return pkm_abi::fail(PKM_EINVAL, "tables and staged must not be NULL");
  if ((((uintptr_t)tables | (uintptr_t)staged) & 15) != 0)
    return pkm_abi::fail(PKM_EINVAL, "tables and staged must be 16-byte aligned");
  if ((rc = pkm::device_ok()) != PKM_OK) return rc;
  const void* view = nullptr;
  if ((rc = pkm_abi::device_view(tables, "tables", &view)) != PKM_OK) return rc;
  a.tables = (const uint8_t*)view;
  a.staged = (uint8_t*)staged;
  return pkm::launch_tokens(cfg->dtype, pkm::PREFETCH, a, (hipStream_t)stream);
}

int engram_forward_staged(const engram_config* cfg, const void* staged, const void* h, int64_t T, void* out,
                          float* e_out, float* alpha_out, void* stream) {
  pkm::EngramArgs a;
  // the hash inputs are not read in this mode: any non-NULL placeholders pass the checks
  static const int32_t dummy_ids = 0;
  static const uint64_t dummy_mult = 1;
  int rc = pkm::prepare(cfg, &dummy_ids, T, 1, nullptr, &dummy_mult, a);
  if (rc != PKM_OK) return rc;
  if (T == 0) return PKM_OK;
  if (!staged || !h || !out) return pkm_abi::fail(PKM_EINVAL, "staged, h and out must not be NULL");
  if ((((uintptr_t)staged | (uintptr_t)h | (uintptr_t)out | (uintptr_t)e_out) & 15) != 0)
    return pkm_abi::fail(PKM_EINVAL, "staged, h, out and e_out must be 16-byte aligned");
  if ((rc = pkm::device_ok()) != PKM_OK) return rc;
  a.ids = nullptr;
  a.mult = nullptr;
  a.staged = (uint8_t*)staged;
  a.h = (const uint8_t*)h;
  a.out = (uint8_t*)out;
  a.e_out = e_out;
  a.alpha_out = alpha_out;
  return pkm::launch_tokens(cfg->dtype, pkm::STAGED, a, (hipStream_t)stream);
}

}  // extern "C"
