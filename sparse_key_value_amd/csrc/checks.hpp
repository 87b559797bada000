// Host-only argument checks of the Engram lookup, the bag backward and the Memory Attention
// values.  Pure C++ (no HIP types or calls), like layout.hpp for the product-key forward, so
// that every check can be built and run on the CPU alone (and under sanitizers).  Each
// returns an empty string if the arguments are valid, else the reason; the entry points turn
// a reason into PKM_EINVAL.  Every product is formed only after its factors are bounded, so no
// check overflows whatever the caller passes.
#pragma once

#include <stdint.h>

#include <string>

#include "../../include/engram.h"
#include "../../include/pkm.h"

namespace pkm {

constexpr int ENGRAM_MAX_ORDER = 8;   // largest n-gram order
constexpr int ENGRAM_MAX_ORDERS = 4;  // orders per lookup
constexpr int ENGRAM_MAX_SPL = 4;     // 16-byte slices of a token per lane (d * sizeof <= 4096 bytes)
// one wave per token: 2^25 tokens of 64 lanes keep a launch within a dispatch's 2^32 work-items
constexpr int64_t ENGRAM_MAX_TOKENS = (int64_t)1 << 25;
constexpr int BAG_MAX = 2048;         // entries per bag of the backward

inline std::string check_engram(const engram_config* c) {
  if (!c) return "config is NULL";
  if (c->dtype != PKM_F32 && c->dtype != PKM_BF16) return "dtype must be PKM_F32 (0) or PKM_BF16 (1)";
  const int64_t eb = c->dtype == PKM_BF16 ? 2 : 4;
  if (c->min_order < 1) return "min_order must be >= 1";
  if (c->n_orders < 1 || c->n_orders > ENGRAM_MAX_ORDERS) return "n_orders must be in [1, 4]";
  if ((int64_t)c->min_order + c->n_orders - 1 > ENGRAM_MAX_ORDER)
    return "the largest order min_order + n_orders - 1 must be <= 8";
  if (c->n_heads < 1 || c->n_heads > 64) return "n_heads must be in [1, 64]";
  if (c->head_dim < 1 || (c->head_dim * eb) % 16 != 0) return "head_dim * sizeof(dtype) must be a positive multiple of 16";
  if ((int64_t)c->n_heads * c->head_dim * eb > 64 * 16 * ENGRAM_MAX_SPL)
    return "n_heads * head_dim * sizeof(dtype) must be <= 4096 bytes";
  if (c->table_rows < 1) return "table_rows must be >= 1";
  if (c->table_rows >= ((int64_t)1 << 31) || (int64_t)c->n_orders * c->n_heads * c->table_rows >= ((int64_t)1 << 31))
    return "n_orders * n_heads * table_rows must be < 2^31 (int32 rows)";
  if (c->vocab < 1) return "vocab must be >= 1";
  if (c->residual != 0 && c->residual != 1) return "residual must be 0 or 1";
  if (!(c->norm_eps >= 0.0f) || c->norm_eps > 1.0f) return "norm_eps must be in [0, 1]";
  return "";
}

inline std::string check_engram_tokens(int64_t T, int64_t seq_len) {
  if (T < 0 || T > ENGRAM_MAX_TOKENS) return "T must be in [0, 2^25]";
  if (seq_len < 1) return "seq_len must be >= 1";
  return "";
}

inline std::string check_bag_sizes(int64_t n_bags, int32_t bag_size, int64_t n_rows) {
  // one block per bag (dw and the update pass): 2^24 blocks of <= 256 lanes keep a launch within
  // the 2^32 work-items of one dispatch
  if (n_bags < 0 || n_bags >= ((int64_t)1 << 24)) return "n_bags must be in [0, 2^24)";
  if (bag_size < 1 || bag_size > BAG_MAX) return "bag_size must be in [1, 2048]";
  if (n_bags * bag_size >= ((int64_t)1 << 31)) return "n_bags * bag_size must be < 2^31";
  if (n_rows < 1 || n_rows >= ((int64_t)1 << 31)) return "n_rows must be in [1, 2^31)";
  return "";
}

inline std::string check_ma_fold(int64_t vocab, int32_t d_v, int32_t n_heads, float eps, int32_t dtype) {
  if (dtype != PKM_F32 && dtype != PKM_BF16) return "dtype must be PKM_F32 or PKM_BF16";
  const int64_t eb = dtype == PKM_BF16 ? 2 : 4;
  if (d_v <= 0 || (d_v * eb) % 16 != 0) return "d_v * sizeof(dtype) must be a positive multiple of 16";
  if (n_heads < 1 || d_v % n_heads != 0 || ((d_v / n_heads) * eb) % 16 != 0)
    return "n_heads must divide d_v with (d_v / n_heads) * sizeof(dtype) a multiple of 16";
  if (vocab < 0 || vocab > ((int64_t)1 << 38) / n_heads) return "vocab * n_heads must be <= 2^38";
  if (!(eps >= 0.0f) || eps > 1.0f) return "eps must be in [0, 1]";
  return "";
}

inline std::string check_ma_values(int64_t vocab, int32_t d_v, int32_t dtype, int64_t T) {
  if (dtype != PKM_F32 && dtype != PKM_BF16) return "dtype must be PKM_F32 or PKM_BF16";
  const int64_t eb = dtype == PKM_BF16 ? 2 : 4;
  if (d_v <= 0 || (d_v * eb) % 16 != 0) return "d_v * sizeof(dtype) must be a positive multiple of 16";
  if (vocab < 1) return "vocab must be >= 1";
  if (T < 0 || T > ((int64_t)1 << 38) / (d_v * eb / 16)) return "T * d_v must be <= 2^38 16-byte slices";
  return "";
}

}  // namespace pkm
