// k x k combine of the two per-half lists, final top-k and softmax.
//
// Cell (a, b) is the key made of sub-key a of the first half and sub-key b of the
// second; its score is s_0[a] + s_1[b] and its flat index a * n_sub + b ("Memory inside
// the model" overview, how it works: the best of the two half lists are combined,
// which finds the right cell among all n_sub x n_sub).  The final top-k is taken under
// (score desc, flat index asc) over all k*k pairs of list positions, and its scores
// are turned into weights by a softmax (digest, core idea: weighted sum of the top-k
// values; overview: weighted average of about thirty values).  The sum is an fp32 add
// of the two fp32 half scores.
//
// One wave per (token, head).  First the two per-half lists: each half's candidates
// (at most cand_slots(k) keys from the scoring kernel, a superset of its top-k, in two
// unsorted lists) are, when both lists hold at most 32 keys, sorted one list per 32-lane half
// by a bitonic network and merged, else ranked by comparing every key with every other
// (v_readlane broadcasts); the k best are written, in order, to LDS (and to the per-half
// outputs when asked for).  Both lists are
// then sorted, so the pair of positions (i, j) is beaten by every (i', j') with i' <= i,
// j' <= j; in exact arithmetic only the "staircase" (i + 1)(j + 1) <= k can reach the
// top-k (119 pairs for k = 32 instead of 1,024).  Staircase cells below a lower bound of
// the k-th best sum are dropped, and the rest sorted with a bitonic network (one key per
// lane when at most 64 are left, else two per lane over all 128 slots).  The
// fp32 rounding of a sum can merge two distinct sums into a tie that the flat index
// then breaks the other way, so the cells off the staircase are checked against the
// k-th key found (one check per row of the grid, by monotonicity); if any could reach
// it (a rounding tie, about never with real data) the wave redoes the selection over
// all k*k pairs.  k = 33..64 (more staircase cells than two per lane: 280 for k = 64) takes
// a kernel of its own that keeps up to five cells per lane and selects the k best by k
// rounds of a wave-wide maximum.
#include "kernels.hpp"

namespace pkm {

namespace {

struct Stair {
  uint16_t pos[128];  // (i << 8) | j for staircase slot s, 0xFFFF = empty
  uint8_t first_off[32];  // row a's first column off the staircase: floor(k / (a + 1))
  uint8_t rect_col[32];   // ceil(k / (a + 1)) - 1: rows 0..a x columns 0..rect_col[a] hold >= k cells
};

// Sort 64 keys held one per lane in descending order (lane 0 ends with the largest).  A
// compare-exchange keeps x when (x > o) matches the side's keep-the-larger flag, else takes o:
// one 64-bit compare and two selects (building both the max and the min took six).
__device__ __forceinline__ uint64_t sort64_desc(uint64_t x, int lane) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint64_t o = shfl_xor_u64(x, stride);
      // keep the larger where bit `size` and bit `stride` of the lane agree (a constant lane mask)
      const bool take_max = lane_in(~(lanes_bit_clear(size) ^ lanes_bit_clear(stride)));
      x = (x > o) == take_max ? x : o;
    }
  }
  return x;
}

// Sort the keys of each 32-lane half of the wave (one per lane) in descending order, the
// two halves independently (lanes 0 and 32 end with their half's largest): the bitonic network
// of sort64_desc up to blocks of 32, whose last merge runs descending in both halves.
__device__ __forceinline__ uint64_t sort32x2_desc(uint64_t x) {
#pragma unroll
  for (int size = 2; size <= 32; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint64_t o = shfl_xor_u64(x, stride);
      const bool take_max = lane_in(~(lanes_bit_clear(size < 32 ? size : 64) ^ lanes_bit_clear(stride)));
      x = (x > o) == take_max ? x : o;
    }
  }
  return x;
}

// Sort 128 keys held two per lane (element e = 2 * lane + slot) in descending order.
__device__ __forceinline__ void sort128_desc(uint64_t& x0, uint64_t& x1, int lane) {
#pragma unroll
  for (int size = 2; size <= 128; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride == 1) {
        // within the lane: elements 2l and 2l+1; block direction from bit `size` of e = 2l
        const bool desc = lane_in(lanes_bit_clear(size >> 1));  // bit `size` of element 2 lane clear
        const bool keep = (x0 > x1) == desc;  // x0 already on its side
        const uint64_t t = x0;
        x0 = keep ? x0 : x1;
        x1 = keep ? x1 : t;
      } else {
        const int lx = stride >> 1;  // partner lane: e ^ stride = 2 * (lane ^ lx) + slot
        const uint64_t o0 = shfl_xor_u64(x0, lx), o1 = shfl_xor_u64(x1, lx);
        // keep the larger where bit `size` of element 2 lane and bit lx of the lane agree
        const bool take_max = lane_in(~(lanes_bit_clear(size >> 1) ^ lanes_bit_clear(lx)));
        x0 = (x0 > o0) == take_max ? x0 : o0;
        x1 = (x1 > o1) == take_max ? x1 : o1;
      }
    }
  }
}

__global__ void __launch_bounds__(256) combine_kernel(const uint64_t* __restrict__ cand,
                                                      const int32_t* __restrict__ count, int64_t rows, int n, int k,
                                                      Stair st, int32_t* __restrict__ half_idx,
                                                      float* __restrict__ half_score, int32_t* __restrict__ idx,
                                                      float* __restrict__ score, float* __restrict__ w) {
  __shared__ uint64_t lists[4][2][32];
  __shared__ uint64_t surv[4][64];
  // the wave index made explicitly uniform: the row, its counts and the ranking loops
  // below are then scalar (a per-lane count made each loop divergent, with exec-mask
  // updates in every iteration)
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;  // row = t * H + h
  if (row >= rows) return;

  // per-half top-k from the candidates, sorted by rank
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    // candidates: lane half 0 in slots [0, 64), half 1 in [64, 128) (cand_slots(k) = 128)
    const int64_t r2 = row * 2 + c;
    const int na = count[2 * r2], nb = count[2 * r2 + 1];  // <= 64 after the overflow pass
    const uint64_t* cr = cand + r2 * 128;
    // Lists of up to 32 keys: lanes 0-31 hold list 0 and lanes 32-63 list 1, each half sorted
    // by a bitonic network (empty slots are key 0 and sort last); a key's rank is then its
    // position in its own list plus the number of the other list's keys above it (a binary
    // search; the keys are distinct).
    if (na <= 32 && nb <= 32) {  // wave-uniform
      const int own = lane & 31, side = lane >> 5;
      const int n_own = side ? nb : na, n_oth = side ? na : nb;
      const uint64_t x = sort32x2_desc(own < n_own ? cr[64 * side + own] : 0ull);
      surv[wv][lane] = x;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      const uint64_t* oth = surv[wv] + 32 * (1 - side);
      int lo = 0, hi = n_oth;
#pragma unroll
      for (int it = 0; it < 6; ++it) {  // n_oth <= 32
        if (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (oth[mid] > x) lo = mid + 1;
          else hi = mid;
        }
      }
      const int rank = own + lo;
      if (own < n_own && rank < k) lists[wv][c][rank] = x;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      continue;
    }
    const uint64_t x0 = lane < na ? cr[lane] : 0ull;
    const uint64_t x1 = lane < nb ? cr[64 + lane] : 0ull;
    // rank = the number of candidates with a larger key; two broadcasts per step so that
    // the compares of one step do not wait on each other's carry
    int r0 = 0, r1 = 0, q0 = 0, q1 = 0;
    int i = 0;
    for (; i + 1 < na; i += 2) {
      const uint64_t y = readlane_u64(x0, i), z = readlane_u64(x0, i + 1);
      r0 += y > x0;
      r1 += y > x1;
      q0 += z > x0;
      q1 += z > x1;
    }
    if (i < na) {
      const uint64_t y = readlane_u64(x0, i);
      r0 += y > x0;
      r1 += y > x1;
    }
    for (i = 0; i + 1 < nb; i += 2) {
      const uint64_t y = readlane_u64(x1, i), z = readlane_u64(x1, i + 1);
      r0 += y > x0;
      r1 += y > x1;
      q0 += z > x0;
      q1 += z > x1;
    }
    if (i < nb) {
      const uint64_t y = readlane_u64(x1, i);
      r0 += y > x0;
      r1 += y > x1;
    }
    r0 += q0;
    r1 += q1;
    if (lane < na && r0 < k) lists[wv][c][r0] = x0;
    if (lane < nb && r1 < k) lists[wv][c][r1] = x1;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  if (half_idx && lane < 2 * k) {  // the per-half lists, when asked for
    const int c = lane / k, j = lane - c * k;
    const uint64_t key = lists[wv][c][j];
    const int64_t o = (row * 2 + c) * k + j;
    half_idx[o] = (int32_t)key_index(key);
    half_score[o] = key_score(key);
  }
  const uint64_t* L0 = lists[wv][0];
  const uint64_t* L1 = lists[wv][1];
  auto cell_key = [&](int a, int b) -> uint64_t {
    return make_key(key_score(L0[a]) + key_score(L1[b]), key_index(L0[a]) * (uint32_t)n + key_index(L1[b]));
  };

  // staircase keys, two per lane
  const uint16_t p0 = st.pos[2 * lane], p1 = st.pos[2 * lane + 1];
  uint64_t x0 = p0 != 0xFFFF ? cell_key(p0 >> 8, p0 & 0xFF) : 0ull;
  uint64_t x1 = p1 != 0xFFFF ? cell_key(p1 >> 8, p1 & 0xFF) : 0ull;
  // A lower bound of the k-th best sum: rows 0..a x columns 0..ceil(k/(a+1))-1 are at
  // least k cells, each summing to at least the corner's sum (sorted lists, monotone fp32
  // add), for every a; the largest such corner bounds the k-th best from below.  Staircase
  // cells below it cannot be among the best k.  When at least k and at most 64 survive
  // (about 70% of rows with random data), they are sorted one per lane; otherwise all
  // 128 slots are, two per lane.
  float lb = lane < k ? key_score(L0[lane]) + key_score(L1[st.rect_col[lane]]) : -__builtin_inff();
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lb = fmaxf(lb, __shfl_xor(lb, o, WAVE));
  const bool keep0 = x0 != 0ull && key_score(x0) >= lb, keep1 = x1 != 0ull && key_score(x1) >= lb;
  const uint64_t m0 = __ballot(keep0), m1 = __ballot(keep1);
  const int ns = __popcll(m0) + __popcll(m1);
  const bool few = ns >= k && ns <= 64;  // wave-uniform
  uint64_t y = 0ull, kth;
  if (few) {
    const uint64_t below = (1ull << lane) - 1ull;  // lanes under this one (lane < 64)
    if (keep0) surv[wv][__popcll(m0 & below)] = x0;
    if (keep1) surv[wv][__popcll(m0) + __popcll(m1 & below)] = x1;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    y = lane < ns ? surv[wv][lane] : 0ull;
    y = sort64_desc(y, lane);
    kth = shfl_u64(y, k - 1);
  } else {
    sort128_desc(x0, x1, lane);
    // element e = 2 * lane + slot; the k-th best is element k - 1
    kth = shfl_u64((k - 1) & 1 ? x1 : x0, (k - 1) >> 1);
  }

  // nothing off the staircase may beat the k-th key.  Both lists are sorted and an fp32
  // add is monotone, so the largest off-staircase sum of row a is at its first
  // off-staircase column b0 = floor(k / (a + 1)): if that sum is below the k-th score, no
  // cell of the row reaches it (a cell can only beat the k-th key by a larger sum, or by
  // an equal sum with a lower flat index).  Lane a checks row a; a row that fails is
  // settled by the exhaustive selection below.
  const float kth_score = key_score(kth);
  bool beaten = false;
  if (lane < k) {
    const int b0 = st.first_off[lane];  // a table: a per-lane integer division costs ~20 VALU ops
    if (b0 < k) beaten = key_score(L0[lane]) + key_score(L1[b0]) >= kth_score;
  }
  uint64_t mine;  // lane j < k ends up with the j-th best key
  if (__ballot(beaten) == 0) {
    if (few) {
      mine = y;
    } else {
      // lane j takes element j = 2 * (j >> 1) + (j & 1)
      const uint64_t a0 = shfl_u64(x0, lane >> 1), a1 = shfl_u64(x1, lane >> 1);
      mine = (lane & 1) ? a1 : a0;
    }
  } else {
    // exhaustive: k rounds of a wave-wide maximum over all k*k keys
    const int kk = k * k;
    uint64_t key[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int cidx = lane + 64 * r;
      key[r] = cidx < kk ? cell_key(cidx / k, cidx % k) : 0ull;
    }
    mine = 0ull;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0ull;
#pragma unroll
      for (int r = 0; r < 16; ++r) best = key[r] > best ? key[r] : best;
      const uint64_t win = wave_max_u64(best);
#pragma unroll
      for (int r = 0; r < 16; ++r) key[r] = key[r] == win ? 0ull : key[r];
      if (lane == j) mine = win;
    }
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

// The staircase of k = 33..64: (i + 1)(j + 1) <= k holds at most 280 cells (k = 64).
struct StairWide {
  uint16_t pos[320];      // (i << 8) | j for slot s (lane s % 64 holds slots s, s + 64, ...), 0xFFFF = empty
  uint8_t first_off[64];  // row a's first column off the staircase: floor(k / (a + 1))
};

// The combine for k = 33..64: per-half ranking over up to 128 candidates per lane half (four
// per lane), the staircase cells five per lane, the k best by k rounds of a wave-wide maximum,
// the off-staircase check with an exhaustive redo, and the softmax.
__global__ void __launch_bounds__(256) combine_wide_kernel(const uint64_t* __restrict__ cand,
                                                           const int32_t* __restrict__ count, int64_t rows, int n,
                                                           int k, StairWide st, int32_t* __restrict__ half_idx,
                                                           float* __restrict__ half_score, int32_t* __restrict__ idx,
                                                           float* __restrict__ score, float* __restrict__ w) {
  constexpr int CS = 256, HALF = CS / 2;  // cand_slots(k) for k > 32
  __shared__ uint64_t lists[4][2][MAX_K];
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;  // row = t * H + h
  if (row >= rows) return;

#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int64_t r2 = row * 2 + c;
    const int na = count[2 * r2], nb = count[2 * r2 + 1];  // <= HALF after the overflow pass
    const uint64_t* cr = cand + r2 * CS;
    // candidate q of this lane: slot lane + 64 q of lane half 0 (q < 2) or of lane half 1
    uint64_t x[4];
    x[0] = lane < na ? cr[lane] : 0ull;
    x[1] = 64 + lane < na ? cr[64 + lane] : 0ull;
    x[2] = lane < nb ? cr[HALF + lane] : 0ull;
    x[3] = 64 + lane < nb ? cr[HALF + 64 + lane] : 0ull;
    // rank = the number of candidates with a larger key (keys are distinct; empty slots are 0)
    int r[4] = {0, 0, 0, 0};
    auto count_above = [&](uint64_t y) {
#pragma unroll
      for (int q = 0; q < 4; ++q) r[q] += y > x[q];
    };
    for (int i = 0; i < na && i < 64; ++i) count_above(readlane_u64(x[0], i));
    for (int i = 64; i < na; ++i) count_above(readlane_u64(x[1], i - 64));
    for (int i = 0; i < nb && i < 64; ++i) count_above(readlane_u64(x[2], i));
    for (int i = 64; i < nb; ++i) count_above(readlane_u64(x[3], i - 64));
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (x[q] != 0ull && r[q] < k) lists[wv][c][r[q]] = x[q];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  if (half_idx) {  // the per-half lists, when asked for
    for (int e = lane; e < 2 * k; e += 64) {
      const int c = e / k, j = e - c * k;
      const uint64_t key = lists[wv][c][j];
      const int64_t o = (row * 2 + c) * k + j;
      half_idx[o] = (int32_t)key_index(key);
      half_score[o] = key_score(key);
    }
  }
  const uint64_t* L0 = lists[wv][0];
  const uint64_t* L1 = lists[wv][1];
  auto cell_key = [&](int a, int b) -> uint64_t {
    return make_key(key_score(L0[a]) + key_score(L1[b]), key_index(L0[a]) * (uint32_t)n + key_index(L1[b]));
  };

  // the staircase cells, five slots per lane; the k best by rounds of a wave-wide maximum
  uint64_t x[5];
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    const uint16_t p = st.pos[lane + 64 * m];
    x[m] = p != 0xFFFF ? cell_key(p >> 8, p & 0xFF) : 0ull;
  }
  uint64_t mine = 0ull, kth = 0ull;  // lane j < k ends up with the j-th best key
  for (int j = 0; j < k; ++j) {
    uint64_t best = x[0];
#pragma unroll
    for (int m = 1; m < 5; ++m) best = x[m] > best ? x[m] : best;
    const uint64_t win = wave_max_u64(best);
#pragma unroll
    for (int m = 0; m < 5; ++m) x[m] = x[m] == win ? 0ull : x[m];
    if (lane == j) mine = win;
    kth = win;
  }

  // nothing off the staircase may beat the k-th key (see the k <= 32 kernel): row a's largest
  // off-staircase sum is at column floor(k / (a + 1)); a row that could reach it sends the
  // wave to an exhaustive selection over all k*k cells, k rounds of a wave-wide maximum
  // below the previous winner (the keys are distinct)
  const float kth_score = key_score(kth);
  bool beaten = false;
  if (lane < k) {
    const int b0 = st.first_off[lane];
    if (b0 < k) beaten = key_score(L0[lane]) + key_score(L1[b0]) >= kth_score;
  }
  if (__ballot(beaten) != 0) {
    uint64_t prev = ~0ull;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0ull;
      for (int a = 0; a < k; ++a) {
        const uint64_t key = lane < k ? cell_key(a, lane) : 0ull;
        best = key < prev && key > best ? key : best;
      }
      const uint64_t win = wave_max_u64(best);
      if (lane == j) mine = win;
      prev = win;
    }
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

}  // namespace

hipError_t launch_combine(const uint64_t* cand, const int32_t* count, int64_t T, int H, int n, int k,
                          int32_t* half_idx, float* half_score, int32_t* idx, float* score, float* w, hipStream_t s) {
  const int64_t rows = T * H;
  if (rows == 0) return hipSuccess;
  if (k > 32) {
    StairWide st;
    int m = 0;
    for (int a = 0; a < k; ++a)
      for (int b = 0; (a + 1) * (b + 1) <= k; ++b) st.pos[m++] = (uint16_t)((a << 8) | b);
    for (; m < 320; ++m) st.pos[m] = 0xFFFF;
    for (int a = 0; a < 64; ++a) st.first_off[a] = (uint8_t)(a < k ? k / (a + 1) : 0);
    combine_wide_kernel<<<dim3((unsigned)((rows + 3) / 4)), 256, 0, s>>>(cand, count, rows, n, k, st, half_idx,
                                                                         half_score, idx, score, w);
    return hipGetLastError();
  }
  Stair st;
  int m = 0;
  for (int a = 0; a < k; ++a)
    for (int b = 0; (a + 1) * (b + 1) <= k; ++b) st.pos[m++] = (uint16_t)((a << 8) | b);
  for (; m < 128; ++m) st.pos[m] = 0xFFFF;
  for (int a = 0; a < 32; ++a) st.first_off[a] = (uint8_t)(a < k ? k / (a + 1) : 0);
  for (int a = 0; a < 32; ++a) st.rect_col[a] = (uint8_t)(a < k ? (k + a) / (a + 1) - 1 : 0);
  combine_kernel<<<dim3((unsigned)((rows + 3) / 4)), 256, 0, s>>>(cand, count, rows, n, k, st, half_idx, half_score,
                                                                  idx, score, w);
  return hipGetLastError();
}

}  // namespace pkm
