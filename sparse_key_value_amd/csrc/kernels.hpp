// Launchers of the product-key memory kernels (host-callable, enqueue only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace pkm {

enum { DT_F32 = 0, DT_BF16 = 1 };

// Selection buffers per row (token, head, half): group maxima and candidate keys.
constexpr int MAX_GROUPS = 128;
constexpr int MAX_K = 64;
// Candidate slots per row: half for each of a token's two lanes in the scoring passes; a
// larger k leaves more candidates above the bound.
constexpr int cand_slots(int k) { return k <= 32 ? 128 : 256; }

// GEMM epilogues: C = A[M,K] * Bt[N,K]^T, fp32 accumulation.
enum {
  EPI_STORE_F32 = 0,    // C -> fp32
  EPI_STORE_DT = 1      // C -> dtype
};

// fp8 copies for the bound pass: dst8 [rows, d] = e4m3(src [rows, d] bf16), and norms [rows] =
// the fp32 norm of every row (nullable); kmax (nullable): the largest norm of every group of
// `group` consecutive rows, [rows / group].
hipError_t launch_fp8_rows(const void* src, uint8_t* dst8, float* norms, int64_t rows, int d, float* kmax, int group,
                           hipStream_t s);
hipError_t launch_transpose(const void* src, void* dst, int rows, int cols, int dtype, hipStream_t s);
// Row r of `rows` is element r % per_tok of token r / per_tok: input at token stride in_ld
// elements (0: per_tok * width, rows back to back).  Output rows back to back, each cut into
// segments of `seg` elements stored in `seg_ld` elements with zeros after them (seg = 0: one
// unpadded segment).
// With q8 (bf16 output, 256-wide segments): also the fp8 copy of the output and the norm of every
// segment, qn [rows * (width / seg)].
hipError_t launch_rownorm(const void* in, int in_is_f32, void* out, int out_dtype, int64_t rows, int width,
                          int norm, float eps, hipStream_t s, int per_tok = 1, int64_t in_ld = 0, int seg = 0,
                          int seg_ld = 0, uint8_t* q8 = nullptr, float* qn = nullptr);
// dst [rows, ld] = src [rows, width] with zeros in columns [width, ld).
hipError_t launch_pad_rows(const void* src, void* dst, int64_t rows, int width, int ld, int dtype, hipStream_t s);
hipError_t launch_gemm(const void* A, const void* Bt, void* C, int64_t M, int N, int K, int dtype, int epi,
                       hipStream_t s);
// The bound pass from fp8 scores (bf16 workloads with 256-wide halves; every pointer NULL: the
// exact bound from the stored type): q8 [T, H, 2, d_h] and k8 [H, 2, n, d_h] OCP e4m3 copies of
// qhat and khat, qn [T, H, 2] the norms of the query halves, kmax [H, 2] the largest sub-key
// norm of every (head, half).
struct Fp8Bound {
  const void* q8 = nullptr;
  const void* k8 = nullptr;
  const float* qn = nullptr;
  const float* kmax = nullptr;
};
// Margin of the fp8 bound in units of |q half| * max |sub-key|: the fp8 rounding error of a score
// has a standard deviation of about 0.0024 of that product with qk-normalised rows.
constexpr float FP8_BOUND_ETA = 0.006f;
constexpr bool fp8_bound_for(int d_h_stored, int dtype) { return dtype == DT_BF16 && d_h_stored == 256; }

// Sub-key scoring: per row (t, h, c) of qhat [T, H, 2, d_h] against khat [H, 2, n, d_h]
// (d_h: the stored, padded width), the candidates of its top-k.  Scratch gmax
// [T*H*2, MAX_GROUPS] fp32, theta [T*H*2]; outputs cand [T*H*2, C] 64-bit keys, C =
// cand_slots(k), and count [T*H*2, 2] (candidates in slots [0, C/2) and [C/2, C); each count
// <= C/2 on return).
hipError_t launch_score_candidates(const void* qhat, const void* khat, int64_t T, int H, int d_h, int n, int k,
                                   int dtype, float* gmax, float* theta, uint64_t* cand, int32_t* count,
                                   const Fp8Bound& fb, hipStream_t s);
// Per-half top-k from the candidates, k x k combine, final top-k and softmax.
// Outputs half_idx/half_score [T, H, 2, k] (both NULL: not written), idx/score/w [T, H, k].
hipError_t launch_combine(const uint64_t* cand, const int32_t* count, int64_t T, int H, int n, int k,
                          int32_t* half_idx, float* half_score, int32_t* idx, float* score, float* w, hipStream_t s);
// Weighted EmbeddingBag: y[b] = sum_j w[b,j] table[idx[b,j]]; y fp32 or dtype.  With z
// (row b at z + b * z_ld, dim elements; fp32, or bf16 if z_bf16 with a bf16 table) it writes
// g[b] = y[b] * silu(z[b]) in dtype instead.
hipError_t launch_gather(const void* table, int64_t n_rows, int dim, int dtype, const int32_t* idx,
                         const float* w, int64_t n_bags, int bag, void* y, int y_dtype_is_table, hipStream_t s,
                         const void* z = nullptr, int64_t z_ld = 0, int z_bf16 = 0);

hipError_t launch_convert_f32(const float* in, void* out, int64_t n, int dtype, hipStream_t s);


}  // namespace pkm
