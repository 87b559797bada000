// Sub-key scoring fused with the per-half top-k.
//
// For each (token t, head h, half c): s[i] = <qhat_c[t, h], khat[h, c, i]> for all
// i < n_sub, and the k best i under (score desc, index asc) ("Memory Layers at Scale"
// digest, product-key search: a key is two sub-keys, so each half is scored against
// sqrt(N) sub-keys; "Memory inside the model" overview, how it works: each half is
// compared with its own list of half-keys and the best ones are kept).
//
// Design for gfx950:
//  * The scores are a dense contraction (tokens x sub-keys x d_h) and run on the matrix
//    cores: v_mfma_f32_32x32x16_bf16 (bf16) or v_mfma_f32_32x32x2f32 (fp32).  The MFMA
//    computes S^T = Khat * Qhat^T, so each lane's 16 accumulators belong to ONE token
//    (column = lane % 32) and 16 sub-keys; the selection threshold is one register.
//  * A block is 4 waves x 32 tokens for one (h, c); chunks of 64 sub-keys are staged
//    through LDS once and shared by the 4 waves, the next chunk being prefetched into
//    registers while the current one is scored.
//  * The scores are never written out.  Each token keeps, in LDS, its current top-k
//    plus a pending list (capacity 64 keys).  A score enters the pending list only if
//    its key beats the token's current k-th best key.  When a tile could overflow the
//    list, the token's keys are sorted across the wave (bitonic, one key per lane) and
//    cut back to k, which raises the threshold.  After the first few chunks almost
//    every score is rejected by one compare.
//  * Keys are 64-bit (ordered score << 32 | ~index), so ties resolve to the lower
//    index with no extra compare and every key is distinct.
//  * Blocks are numbered so that block b works on pair (h, c) = b mod 2H; blocks are
//    dealt round-robin to the 8 XCDs, so with 2H dividing 8 each XCD only ever reads
//    one pair's sub-keys, which stay resident in that XCD's L2.
#include "kernels.hpp"

namespace pkm {

namespace {

constexpr int TPW = 32;         // tokens per wave
constexpr int NWAVES = 4;
constexpr int TPB = TPW * NWAVES;
constexpr int CHUNK = 64;       // sub-keys per LDS chunk (two 32-row MFMA tiles)
constexpr int CAP = 64;         // keys per token in the LDS candidate list

template <typename DT, int DH>
struct Mma;

// bf16: A = 32 sub-keys x 16 dims (lane: row l%32, dims (l/32)*8..+7), B = 16 dims x 32 tokens.
template <int DH>
struct Mma<uint16_t, DH> {
  static constexpr int KSTEP = 16;
  static constexpr int NK = DH / KSTEP;
  static constexpr int EB = 2;
  typedef bf16x8 frag;
  __device__ static frag load_q(const uint16_t* q, int kk, int hi) {
    return *(const bf16x8*)(q + kk * KSTEP + hi * 8);
  }
  __device__ static frag lds_k(const uint8_t* row, int kk, int hi) {
    return *(const bf16x8*)(row + (kk * KSTEP + hi * 8) * EB);
  }
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }
};

// fp32: A = 32 sub-keys x 2 dims (lane: row l%32, dim l/32), B = 2 dims x 32 tokens.
template <int DH>
struct Mma<float, DH> {
  static constexpr int KSTEP = 2;
  static constexpr int NK = DH / KSTEP;
  static constexpr int EB = 4;
  typedef float frag;
  __device__ static frag load_q(const float* q, int kk, int hi) { return q[kk * KSTEP + hi]; }
  __device__ static frag lds_k(const uint8_t* row, int kk, int hi) {
    return *(const float*)(row + (kk * KSTEP + hi) * EB);
  }
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0); }
};

// Sort token jj's list across the wave, keep its best k, and update that token's
// count and threshold (held by lanes jj and jj + 32).
__device__ __forceinline__ void merge_token(uint64_t* cand_wave, int jj, int lane, int tok, int k, int& cnt,
                                            uint64_t& thr) {
  __builtin_amdgcn_wave_barrier();
  const int cj = __shfl(cnt, jj, WAVE);
  uint64_t* b = cand_wave + jj * CAP;
  uint64_t key = lane < cj ? b[lane] : 0ull;
  key = wave_sort_desc(key, lane);
  const uint64_t kth = shfl_u64(key, k - 1);
  __builtin_amdgcn_wave_barrier();
  if (lane < k) b[lane] = key;
  __builtin_amdgcn_wave_barrier();
  const int nc = cj < k ? cj : k;
  if (tok == jj) {
    cnt = nc;
    thr = nc >= k ? kth : 0ull;
  }
}

// Offer one 32-sub-key tile of scores (this lane: 16 sub-keys of token `tok`).
__device__ __forceinline__ void offer_tile(const f32x16& acc, int sub_base, int n, int lane, int tok, int hi, int k,
                                           uint64_t* cand_wave, int& cnt, uint64_t& thr) {
  uint64_t key[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int sub = sub_base + 8 * (r >> 2) + 4 * hi + (r & 3);
    key[r] = sub < n ? make_key(acc[r], (uint32_t)sub) : 0ull;
  }
  uint32_t m = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) m |= (key[r] > thr ? 1u : 0u) << r;
  int c = __popc(m);
  int co = __shfl_xor(c, 32, WAVE);
  const bool need = cnt + c + co > CAP;
  uint64_t bal = __ballot(need) & 0xFFFFFFFFull;
  if (bal) {
    while (bal) {
      const int jj = __builtin_ctzll(bal);
      bal &= bal - 1;
      merge_token(cand_wave, jj, lane, tok, k, cnt, thr);
    }
    m = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) m |= (key[r] > thr ? 1u : 0u) << r;
    c = __popc(m);
    co = __shfl_xor(c, 32, WAVE);
  }
  int off = cnt + (hi ? co : 0);
  uint64_t* b = cand_wave + tok * CAP;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (m & (1u << r)) b[off++] = key[r];
  }
  cnt += c + co;
}

template <typename DT, int DH>
__global__ void __launch_bounds__(256) score_topk_kernel(const DT* __restrict__ qhat, const DT* __restrict__ khat,
                                                         int64_t T, int H, int n, int k, int32_t* __restrict__ half_idx,
                                                         float* __restrict__ half_score) {
  using M = Mma<DT, DH>;
  constexpr int RB = DH * M::EB;          // bytes per sub-key row
  constexpr int RS = RB + 16;             // padded LDS row stride
  constexpr int U16 = RB / 16;            // 16-byte units per row
  constexpr int UPT = CHUNK * U16 / 256;  // units per thread per chunk
  static_assert(UPT >= 1 && CHUNK * U16 % 256 == 0, "chunk must split evenly over 256 threads");

  __shared__ __attribute__((aligned(16))) uint8_t ks[CHUNK * RS];
  __shared__ uint64_t cand[TPB * CAP];

  const int pairs = 2 * H;
  const int pair = blockIdx.x % pairs;
  const int64_t tile = blockIdx.x / pairs;
  const int h = pair >> 1, c = pair & 1;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tok = lane & 31, hi = lane >> 5;
  const int64_t t = tile * TPB + wv * TPW + tok;

  // this lane's query fragment (token t, half c, head h); zero past the last token
  typename M::frag qf[M::NK];
  {
    const DT* qrow = qhat + ((t * H + h) * 2 + c) * (int64_t)DH;
#pragma unroll
    for (int kk = 0; kk < M::NK; ++kk) {
      if (t < T) qf[kk] = M::load_q(qrow, kk, hi);
      else qf[kk] = typename M::frag{};
    }
  }

  const uint8_t* kbase = (const uint8_t*)(khat + (size_t)pair * n * DH);
  const int nch = (n + CHUNK - 1) / CHUNK;
  u32x4 pre[UPT];
  auto fetch = [&](int ch) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * 256;
      const int row = u / U16, col = u - row * U16;
      const int sub = ch * CHUNK + row;
      pre[i] = sub < n ? *(const u32x4*)(kbase + (size_t)sub * RB + col * 16) : u32x4{0, 0, 0, 0};
    }
  };
  fetch(0);

  uint64_t* cand_wave = cand + wv * TPW * CAP;
  int cnt = 0;
  uint64_t thr = 0ull;

  for (int ch = 0; ch < nch; ++ch) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * 256;
      const int row = u / U16, col = u - row * U16;
      *(u32x4*)(ks + row * RS + col * 16) = pre[i];
    }
    __syncthreads();
    if (ch + 1 < nch) fetch(ch + 1);

    f32x16 acc0 = {}, acc1 = {};
    const uint8_t* r0 = ks + (lane & 31) * RS;
    const uint8_t* r1 = ks + (32 + (lane & 31)) * RS;
#pragma unroll
    for (int kk = 0; kk < M::NK; ++kk) {
      acc0 = M::mma(M::lds_k(r0, kk, hi), qf[kk], acc0);
      acc1 = M::mma(M::lds_k(r1, kk, hi), qf[kk], acc1);
    }
    offer_tile(acc0, ch * CHUNK, n, lane, tok, hi, k, cand_wave, cnt, thr);
    offer_tile(acc1, ch * CHUNK + 32, n, lane, tok, hi, k, cand_wave, cnt, thr);
  }

  // final sort of every token of this wave, then write its top-k
  for (int jj = 0; jj < TPW; ++jj) {
    const int cj = __shfl(cnt, jj, WAVE);
    uint64_t* b = cand_wave + jj * CAP;
    __builtin_amdgcn_wave_barrier();
    uint64_t key = lane < cj ? b[lane] : 0ull;
    key = wave_sort_desc(key, lane);
    const int64_t tj = tile * TPB + wv * TPW + jj;
    if (tj < T && lane < k) {
      const int64_t o = ((tj * H + h) * 2 + c) * (int64_t)k + lane;
      half_idx[o] = (int32_t)key_index(key);
      half_score[o] = key_score(key);
    }
  }
}

template <typename DT, int DH>
hipError_t launch_st(const void* qhat, const void* khat, int64_t T, int H, int n, int k, int32_t* hi, float* hs,
                     hipStream_t s) {
  const int64_t tiles = (T + TPB - 1) / TPB;
  const int64_t blocks = tiles * 2 * H;
  score_topk_kernel<DT, DH><<<dim3((unsigned)blocks), 256, 0, s>>>((const DT*)qhat, (const DT*)khat, T, H, n, k, hi, hs);
  return hipGetLastError();
}

}  // namespace

bool score_topk_supported(int d_h, int dtype) {
  (void)dtype;
  return d_h == 64 || d_h == 128 || d_h == 256;
}

hipError_t launch_score_topk(const void* qhat, const void* khat, int64_t T, int H, int d_h, int n, int k, int dtype,
                             int32_t* half_idx, float* half_score, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == DT_BF16) {
    switch (d_h) {
      case 64: return launch_st<uint16_t, 64>(qhat, khat, T, H, n, k, half_idx, half_score, s);
      case 128: return launch_st<uint16_t, 128>(qhat, khat, T, H, n, k, half_idx, half_score, s);
      case 256: return launch_st<uint16_t, 256>(qhat, khat, T, H, n, k, half_idx, half_score, s);
    }
  } else {
    switch (d_h) {
      case 64: return launch_st<float, 64>(qhat, khat, T, H, n, k, half_idx, half_score, s);
      case 128: return launch_st<float, 128>(qhat, khat, T, H, n, k, half_idx, half_score, s);
      case 256: return launch_st<float, 256>(qhat, khat, T, H, n, k, half_idx, half_score, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace pkm
