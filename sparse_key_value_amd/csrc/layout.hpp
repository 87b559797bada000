// Host-only: validation of a pkm_config and the carving of the workspace.
// Pure C++ (no HIP calls), so every check runs before the device is touched.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/pkm.h"

namespace pkm {

struct Layout {
  // With the Memory+ gate, W1^T follows W_q^T in one [H d_q + d_v, d_model] matrix and one
  // GEMM computes x [W_q | W1] into the rows of q: columns [0, H d_q) are the query,
  // [H d_q, H d_q + d_v) are z = x W1 (qz_cols columns per token).
  size_t wqT = 0, khat = 0, w1T = 0, w2T = 0;        // create-time copies
  int64_t qz_cols = 0;
  size_t q = 0, qhat = 0, hidx = 0, hsc = 0;          // per-forward intermediates
  size_t gmax = 0, theta = 0, cand = 0, count = 0;    // selection scratch
  // the bound pass from fp8 scores (fp8_bound): e4m3 copies of the sub-keys and the query
  // halves, the sub-key row norms and their largest per (head, half), the query half norms
  size_t khat8 = 0, knorm = 0, kmax = 0, q8 = 0, qn = 0;
  size_t idx = 0, sc = 0, w = 0, g = 0;
  size_t total = 0;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Returns an empty string if the config is valid, else the reason.
inline std::string check_config(const pkm_config* c) {
  if (!c) return "config is NULL";
  if (c->dtype != PKM_F32 && c->dtype != PKM_BF16) return "dtype must be PKM_F32 (0) or PKM_BF16 (1)";
  const int eb = c->dtype == PKM_BF16 ? 2 : 4;
  const int vec = 16 / eb;  // elements per 16-byte access
  if (c->d_model <= 0 || c->d_model % vec != 0)
    return "d_model must be positive and a multiple of " + std::to_string(vec) + " (16-byte rows)";
  if (c->dtype == PKM_BF16 && c->d_model % 32 != 0) return "d_model must be a multiple of 32 for bf16 (GEMM K-tile)";
  if (c->dtype == PKM_BF16 && c->memory_plus && c->d_value % 32 != 0)
    return "d_value must be a multiple of 32 for the bf16 Memory+ gate (GEMM K-tile)";
  // the weight transposes at create tile d_model and d_value on a launch grid's y dimension,
  // which holds at most 65,536 blocks (of 32 rows each here: any width up to 65,536 fits)
  if (c->d_model > 65536) return "d_model must be <= 65536";
  if (c->n_heads < 1 || c->n_heads > 64) return "n_heads must be in [1, 64]";
  if (c->d_query <= 0 || c->d_query % 2 != 0) return "d_query must be positive and even";
  if (c->n_sub < 1) return "n_sub must be >= 1";
  if ((int64_t)c->n_sub * (int64_t)c->n_sub >= ((int64_t)1 << 31)) return "n_sub^2 must be < 2^31 (int32 flat index)";
  if (c->k < 1 || c->k > 64 || c->k > c->n_sub) return "k must satisfy 1 <= k <= min(n_sub, 64)";
  if (c->d_value <= 0 || ((int64_t)c->d_value * eb) % 16 != 0)
    return "d_value * sizeof(dtype) must be a positive multiple of 16";
  if (c->d_value > 65536) return "d_value must be <= 65536";
  if (c->qk_norm != 0 && c->qk_norm != 1) return "qk_norm must be 0 or 1";
  if (c->memory_plus != 0 && c->memory_plus != 1) return "memory_plus must be 0 or 1";
  if (!(c->norm_eps >= 0.0f) || c->norm_eps > 1.0f) return "norm_eps must be in [0, 1]";
  if (c->max_tokens < 1 || c->max_tokens > ((int64_t)1 << 24)) return "max_tokens must be in [1, 2^24]";
  // the selection kernels run one wave per (token, head, half): 2^25 rows of 64 lanes keep a
  // launch within the 2^32 work-items of one dispatch
  if (c->max_tokens * c->n_heads > ((int64_t)1 << 24)) return "max_tokens * n_heads must be <= 2^24";
  return "";
}

// Widest query half the scoring kernels take (d_query <= 512); a valid config beyond it is
// refused with PKM_EUNSUPPORTED rather than PKM_EINVAL.
constexpr int MAX_HALF = 256;

// Returns an empty string if the kernels are built for a valid config, else the reason.
inline std::string unsupported_reason(const pkm_config* c) {
  if (c->d_query / 2 > MAX_HALF) return "d_query / 2 must be <= 256 (the widest query half the scoring kernels hold)";
  return "";
}

// Width of a query half and a sub-key row as stored for scoring: d_query / 2 padded with zeros
// to the next width the scoring kernels are built for (64, 128 or 256).  Zero products leave
// every fp32 dot product unchanged.
inline int padded_half(int d_h) { return d_h <= 64 ? 64 : (d_h <= 128 ? 128 : 256); }

// Whether the bound pass scores in fp8: bf16 workloads whose halves are stored 256 wide.
inline bool fp8_bound(const pkm_config* c) { return c->dtype == PKM_BF16 && padded_half(c->d_query / 2) == 256; }

inline Layout make_layout(const pkm_config* c) {
  Layout L;
  const size_t eb = c->dtype == PKM_BF16 ? 2 : 4;
  const size_t H = c->n_heads, dq = c->d_query, dm = c->d_model, dv = c->d_value, n = c->n_sub, k = c->k;
  const size_t dhp = (size_t)padded_half(c->d_query / 2);
  const size_t T = (size_t)c->max_tokens;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.qz_cols = (int64_t)(H * dq + (c->memory_plus ? dv : 0));
  L.wqT = take((size_t)L.qz_cols * dm * eb);
  if (c->memory_plus) L.w1T = L.wqT + H * dq * dm * eb;
  L.khat = take(H * 2 * n * dhp * eb);
  if (c->memory_plus) L.w2T = take(dm * dv * eb);
  L.q = take(T * (size_t)L.qz_cols * eb);
  L.qhat = take(T * H * 2 * dhp * eb);
  L.gmax = take(T * H * 2 * 128 * 4);   // MAX_GROUPS group maxima per row
  L.theta = take(T * H * 2 * 4);
  L.cand = take(T * H * 2 * (k <= 32 ? 128 : 256) * 8);   // candidate keys per row (cand_slots)
  L.count = take(T * H * 2 * 2 * 4);   // candidates per lane half
  L.hidx = take(T * H * 2 * k * 4);
  L.hsc = take(T * H * 2 * k * 4);
  L.idx = take(T * H * k * 4);
  L.sc = take(T * H * k * 4);
  L.w = take(T * H * k * 4);
  if (c->memory_plus) L.g = take(T * dv * eb);   // y * silu(x W1), the input of the W2 product
  if (fp8_bound(c)) {
    L.khat8 = take(H * 2 * n * dhp);
    L.knorm = take(H * 2 * n * 4);
    L.kmax = take(H * 2 * 4);
    L.q8 = take(T * H * 2 * dhp);
    L.qn = take(T * H * 2 * 4);
  }
  L.total = off;
  return L;
}

}  // namespace pkm
