// k x k combine of the two per-half lists, final top-k and softmax.
//
// Cell (a, b) is the key made of sub-key a of the first half and sub-key b of the
// second; its score is s_0[a] + s_1[b] and its flat index a * n_sub + b ("Memory inside
// the model" overview, how it works: the best of the two half lists are combined,
// which finds the right cell among all n_sub x n_sub).  The final top-k is taken under
// (score desc, flat index asc) and its scores are turned into weights by a softmax
// (digest, core idea: weighted sum of the top-k values; overview: weighted average of
// about thirty values).
//
// One wave per (token, head): each lane forms up to 16 of the k*k <= 1024 candidate
// keys; k rounds of a wave-wide max pull the winners out in order.  The sum is an fp32
// add of the two fp32 half scores.
#include "kernels.hpp"

namespace pkm {

__global__ void __launch_bounds__(256) combine_kernel(const int32_t* __restrict__ half_idx,
                                                      const float* __restrict__ half_score, int64_t rows, int n,
                                                      int k, int32_t* __restrict__ idx, float* __restrict__ score,
                                                      float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // row = t * H + h
  if (row >= rows) return;
  const int32_t* i0 = half_idx + row * 2 * k;
  const int32_t* i1 = i0 + k;
  const float* s0 = half_score + row * 2 * k;
  const float* s1 = s0 + k;

  const int kk = k * k;
  uint64_t key[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int cidx = lane + 64 * r;
    if (cidx < kk) {
      const int a = cidx / k, b = cidx - a * k;
      const float sc = s0[a] + s1[b];
      const uint32_t flat = (uint32_t)i0[a] * (uint32_t)n + (uint32_t)i1[b];
      key[r] = make_key(sc, flat);
    } else {
      key[r] = 0ull;
    }
  }

  uint64_t mine = 0ull;  // lane j < k ends up holding the j-th best key
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0ull;
#pragma unroll
    for (int r = 0; r < 16; ++r) best = key[r] > best ? key[r] : best;
    const uint64_t win = wave_max_u64(best);
#pragma unroll
    for (int r = 0; r < 16; ++r) key[r] = key[r] == win ? 0ull : key[r];
    if (lane == j) mine = win;
  }

  // softmax over the k winners (max = the first one)
  const float top = key_score(shfl_u64(mine, 0));
  const float sc = key_score(mine);
  const float e = lane < k ? __expf(sc - top) : 0.f;
  const float z = wave_sum_f32(e);
  if (lane < k) {
    const int64_t o = row * k + lane;
    idx[o] = (int32_t)key_index(mine);
    score[o] = sc;
    w[o] = e / z;
  }
}

hipError_t launch_combine(const int32_t* half_idx, const float* half_score, int64_t T, int H, int n, int k,
                          int32_t* idx, float* score, float* w, hipStream_t s) {
  const int64_t rows = T * H;
  if (rows == 0) return hipSuccess;
  combine_kernel<<<dim3((unsigned)((rows + 3) / 4)), 256, 0, s>>>(half_idx, half_score, rows, n, k, idx, score, w);
  return hipGetLastError();
}

}  // namespace pkm
