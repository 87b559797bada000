// Launchers of the product-key memory kernels (host-callable, enqueue only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace pkm {

enum { DT_F32 = 0, DT_BF16 = 1 };

// Selection buffers per row (token, head, half): group maxima and candidate keys.
constexpr int MAX_GROUPS = 128;
constexpr int CAND = 128;

// GEMM epilogues: C = A[M,K] * Bt[N,K]^T, fp32 accumulation.
enum {
  EPI_STORE_F32 = 0,    // C -> fp32
  EPI_STORE_DT = 1      // C -> dtype
};

hipError_t launch_transpose(const void* src, void* dst, int rows, int cols, int dtype, hipStream_t s);
// Row r of `rows` is element r % per_tok of token r / per_tok: input at token stride in_ld
// elements (0: per_tok * width, rows back to back), output rows back to back.
hipError_t launch_rownorm(const void* in, int in_is_f32, void* out, int out_dtype, int64_t rows, int width,
                          int norm, float eps, hipStream_t s, int per_tok = 1, int64_t in_ld = 0);
hipError_t launch_gemm(const void* A, const void* Bt, void* C, int64_t M, int N, int K, int dtype, int epi,
                       hipStream_t s);
// Sub-key scoring: per row (t, h, c) of qhat [T, H, 2, d_h] against khat [H, 2, n, d_h],
// the candidates of its top-k.  Scratch gmax [T*H*2, MAX_GROUPS] fp32, theta [T*H*2];
// outputs cand [T*H*2, CAND] 64-bit keys and count [T*H*2, 2] (candidates in slots
// [0, CAND/2) and [CAND/2, CAND); each count <= CAND/2 on return).
hipError_t launch_score_candidates(const void* qhat, const void* khat, int64_t T, int H, int d_h, int n, int k,
                                   int dtype, float* gmax, float* theta, uint64_t* cand, int32_t* count,
                                   hipStream_t s);
// Per-half top-k from the candidates, k x k combine, final top-k and softmax.
// Outputs half_idx/half_score [T, H, 2, k] (both NULL: not written), idx/score/w [T, H, k].
hipError_t launch_combine(const uint64_t* cand, const int32_t* count, int64_t T, int H, int n, int k,
                          int32_t* half_idx, float* half_score, int32_t* idx, float* score, float* w, hipStream_t s);
// Weighted EmbeddingBag: y[b] = sum_j w[b,j] table[idx[b,j]]; y fp32 or dtype.  With z
// (fp32, row b at z + b * z_ld, dim elements) it writes g[b] = y[b] * silu(z[b]) in dtype
// instead.  persistent: a grid of two blocks per CU (for running beside other kernels).
hipError_t launch_gather(const void* table, int64_t n_rows, int dim, int dtype, const int32_t* idx,
                         const float* w, int64_t n_bags, int bag, void* y, int y_dtype_is_table, hipStream_t s,
                         const float* z = nullptr, bool persistent = false, int64_t z_ld = 0);

hipError_t launch_convert_f32(const float* in, void* out, int64_t n, int dtype, hipStream_t s);

bool score_topk_supported(int d_h, int dtype);

}  // namespace pkm
