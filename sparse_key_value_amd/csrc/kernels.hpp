// Launchers of the product-key memory kernels (host-callable, enqueue only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace pkm {

enum { DT_F32 = 0, DT_BF16 = 1 };

// GEMM epilogues: C = A[M,K] * Bt[N,K]^T, fp32 accumulation.
enum {
  EPI_STORE_F32 = 0,    // C -> fp32
  EPI_STORE_DT = 1,     // C -> dtype
  EPI_GATE = 2          // dtype(aux[m,n] * silu(C)), aux fp32 [M, N]
};

hipError_t launch_transpose(const void* src, void* dst, int rows, int cols, int dtype, hipStream_t s);
hipError_t launch_rownorm(const void* in, int in_is_f32, void* out, int out_dtype, int64_t rows, int width,
                          int norm, float eps, hipStream_t s);
hipError_t launch_gemm(const void* A, const void* Bt, void* C, const float* aux, int64_t M, int N, int K,
                       int dtype, int epi, hipStream_t s);
// Fused sub-key scoring and per-half top-k.  qhat [T, H, 2, d_h], khat [H, 2, n, d_h];
// outputs [T, H, 2, k].
hipError_t launch_score_topk(const void* qhat, const void* khat, int64_t T, int H, int d_h, int n, int k,
                             int dtype, int32_t* half_idx, float* half_score, hipStream_t s);
// k x k combine, final top-k and softmax; outputs [T, H, k].
hipError_t launch_combine(const int32_t* half_idx, const float* half_score, int64_t T, int H, int n, int k,
                          int32_t* idx, float* score, float* w, hipStream_t s);
// Weighted EmbeddingBag: y[b] = sum_j w[b,j] table[idx[b,j]]; y fp32 or dtype.
hipError_t launch_gather(const void* table, int64_t n_rows, int dim, int dtype, const int32_t* idx,
                         const float* w, int64_t n_bags, int bag, void* y, int y_dtype_is_table, hipStream_t s);

hipError_t launch_convert_f32(const float* in, void* out, int64_t n, int dtype, hipStream_t s);

bool score_topk_supported(int d_h, int dtype);

}  // namespace pkm
