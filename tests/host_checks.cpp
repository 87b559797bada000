// Host-side argument checks and workspace layout of the library, built on their own (no HIP)
// so that a test can run them under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Reads one case per line from stdin and prints one verdict per line:
//   pkm d_model n_heads d_query n_sub k d_value dtype qk_norm memory_plus norm_eps max_tokens
//       -> "ok <workspace bytes>" | "einval <reason>" | "eunsupported <reason>"
//   engram min_order n_orders n_heads head_dim table_rows vocab dtype residual norm_eps T seq_len
//   bag n_bags bag_size n_rows
//   mafold vocab d_v n_heads eps dtype
//   mavalues vocab d_v dtype T
//       -> "ok" | "einval <reason>"
#include <stdio.h>
#include <stdlib.h>

#include <iostream>
#include <sstream>
#include <string>

#include "checks.hpp"
#include "layout.hpp"

namespace {

// The next field of the line: integers by strtoll, floats by strtof (which reads "nan" and "inf").
struct Fields {
  std::istringstream in;
  explicit Fields(const std::string& line) : in(line) {}
  std::string word() {
    std::string w;
    in >> w;
    return w;
  }
  int64_t i64() { return strtoll(word().c_str(), nullptr, 10); }
  int32_t i32() { return (int32_t)i64(); }
  float f32() { return strtof(word().c_str(), nullptr); }
};

void verdict(const std::string& why, const char* code = "einval") {
  if (why.empty())
    std::cout << "ok\n";
  else
    std::cout << code << " " << why << "\n";
}

}  // namespace

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    Fields f(line);
    const std::string kind = f.word();
    if (kind == "pkm") {
      pkm_config c{};
      c.d_model = f.i32();
      c.n_heads = f.i32();
      c.d_query = f.i32();
      c.n_sub = f.i32();
      c.k = f.i32();
      c.d_value = f.i32();
      c.dtype = f.i32();
      c.qk_norm = f.i32();
      c.memory_plus = f.i32();
      c.norm_eps = f.f32();
      c.max_tokens = f.i64();
      std::string why = pkm::check_config(&c);
      if (!why.empty()) {
        verdict(why);
        continue;
      }
      why = pkm::unsupported_reason(&c);
      if (!why.empty()) {
        verdict(why, "eunsupported");
        continue;
      }
      std::cout << "ok " << pkm::make_layout(&c).total << "\n";
    } else if (kind == "engram") {
      engram_config c{};
      c.min_order = f.i32();
      c.n_orders = f.i32();
      c.n_heads = f.i32();
      c.head_dim = f.i32();
      c.table_rows = f.i64();
      c.vocab = f.i32();
      c.dtype = f.i32();
      c.residual = f.i32();
      c.norm_eps = f.f32();
      const int64_t T = f.i64(), seq_len = f.i64();
      std::string why = pkm::check_engram(&c);
      if (why.empty()) why = pkm::check_engram_tokens(T, seq_len);
      verdict(why);
    } else if (kind == "bag") {
      const int64_t n_bags = f.i64();
      const int32_t bag = f.i32();
      const int64_t n_rows = f.i64();
      verdict(pkm::check_bag_sizes(n_bags, bag, n_rows));
    } else if (kind == "mafold") {
      const int64_t vocab = f.i64();
      const int32_t d_v = f.i32(), n_heads = f.i32();
      const float eps = f.f32();
      const int32_t dtype = f.i32();
      verdict(pkm::check_ma_fold(vocab, d_v, n_heads, eps, dtype));
    } else if (kind == "mavalues") {
      const int64_t vocab = f.i64();
      const int32_t d_v = f.i32(), dtype = f.i32();
      const int64_t T = f.i64();
      verdict(pkm::check_ma_values(vocab, d_v, dtype, T));
    } else if (!kind.empty()) {
      std::cerr << "unknown case: " << line << "\n";
      return 2;
    }
  }
  return 0;
}
