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
//  * A block is 4 waves x 32 tokens for one (h, c).  Chunks of 32 sub-keys are staged
//    through LDS (XOR-swizzled 16-byte units, so the MFMA operand reads are free of
//    bank conflicts without padding) and shared by the 4 waves; the next chunk is
//    prefetched into registers while the current one is scored.  80 KiB of LDS per
//    block lets two blocks share a CU, so one block's selection work overlaps the
//    other's matrix work.
//  * The scores are never written out.  Selection takes two passes over the sub-keys.
//    Pass 1 keeps, per token, the maximum score of each group of sub-keys (at most 128
//    groups); the k-th largest of these maxima is reached by at least k sub-keys, so it
//    bounds the token's k-th best score from below (found bit by bit with wave
//    ballots).  Pass 2 recomputes the same scores and keeps only those at or above the
//    bound: with random-like data about 37 of 4,096 per token.
//  * Each token owns 64 LDS slots of 64-bit keys: pending keys, and after a merge a
//    sorted list in slots 0..31 with pending keys in 32..63.  After a merge a score
//    must beat the k-th best score strictly (every later sub-key has a higher index,
//    so a tie never enters).  A merge is done by the whole wave: each lane ranks its
//    key by comparing it with every key of the token (LDS broadcast reads, no
//    dependent shuffle chain) and ds_permute moves every key to the lane of its rank.
//  * Keys are 64-bit (ordered score << 32 | ~index): ties resolve to the lower index
//    and every key is distinct.  Empty slots carry their lane number, below any key.
//  * Blocks are numbered so that block b works on pair (h, c) = b mod 2H; blocks are
//    dealt round-robin to the 8 XCDs, so with 2H dividing 8 each XCD only ever reads
//    one pair's sub-keys, which stay resident in that XCD's L2.
#include "kernels.hpp"

namespace pkm {

namespace {

constexpr int TPW = 32;         // tokens per wave
constexpr int NWAVES = 4;
constexpr int TPB = TPW * NWAVES;
constexpr int CHUNK = 32;       // sub-keys per LDS chunk (one 32-row MFMA tile)
constexpr int SLOTS = 64;       // keys per token: 32 list + 32 pending
constexpr int LIST = 32;

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
  // operand of k-step kk for this lane: 16-byte unit 2*kk + hi of the lane's row
  __device__ static frag lds_k(const uint8_t* row, int swz, int kk, int hi) {
    return *(const bf16x8*)(row + (((2 * kk + hi) ^ swz) << 4));
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
  __device__ static frag lds_k(const uint8_t* row, int swz, int kk, int hi) {
    const int e = kk * KSTEP + hi;  // element; 4 per 16-byte unit
    return *(const float*)(row + ((((e >> 2) ^ swz) << 4) | ((e & 3) << 2)));
  }
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0); }
};

__device__ __forceinline__ uint64_t permute_u64(uint64_t v, int dst_lane) {
  const int addr = dst_lane << 2;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_permute(addr, (int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_permute(addr, (int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Largest float strictly below x (finite x): "s > below(x)" is "s >= x".
__device__ __forceinline__ float float_below(float x) {
  const uint32_t b = __float_as_uint(x);
  if ((b & 0x7FFFFFFFu) == 0) return __uint_as_float(0x80000001u);
  return __uint_as_float((b & 0x80000000u) ? b + 1 : b - 1);
}

// Per-token selection state, held by the two lanes that own the token.
struct TokState {
  int nl;      // keys in the sorted list (slots 0..nl-1); 0 until the first merge
  int np;      // pending keys, from slot pbase(): all 64 slots are pending until a list exists
  float thr;   // a score must be > thr to be pending
  __device__ int pbase() const { return nl ? LIST : 0; }
  __device__ int cap() const { return nl ? SLOTS - LIST : SLOTS; }
};

// Merge token jj's list and pending keys with the whole wave, leaving the best
// min(32, nl + np) keys sorted in slots 0.. .  Each lane ranks its key by comparing it
// with every real key of the token (LDS broadcast reads, no cross-lane dependency
// chain); ds_permute then sends every key to the lane of its rank.  Keys are distinct,
// so the ranks of the real keys are 0 .. nl+np-1.
__device__ __forceinline__ void merge_token(uint64_t* cand_wave, int jj, int lane, int tok, int k, TokState& st) {
  __builtin_amdgcn_wave_barrier();
  const int nl = __builtin_amdgcn_readlane(st.nl, jj);
  const int np = __builtin_amdgcn_readlane(st.np, jj);
  const int pb = nl ? LIST : 0;
  uint64_t* b = cand_wave + jj * SLOTS;
  const bool real = lane < nl || (lane >= pb && lane - pb < np);
  const uint64_t key = real ? b[lane] : 0ull;
  int rank = 0;
  for (int i = 0; i < nl; ++i) rank += b[i] > key ? 1 : 0;
  for (int i = 0; i < np; ++i) rank += b[pb + i] > key ? 1 : 0;
  const uint64_t sorted = permute_u64(key, real ? rank : SLOTS - 1);
  const int total = nl + np;
  __builtin_amdgcn_wave_barrier();
  if (lane < LIST && lane < total) b[lane] = sorted;
  __builtin_amdgcn_wave_barrier();
  const int nn = total < LIST ? total : LIST;
  const uint32_t kth_ord = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(sorted >> 32), k - 1);
  if (tok == jj) {
    st.nl = nn;
    st.np = 0;
    // once k keys are listed, a later sub-key (higher index) must beat the k-th score strictly
    if (nn >= k) st.thr = score_of_ord(kth_ord);
  }
}

__device__ __forceinline__ int sub_of(int sub_base, int r, int hi) { return sub_base + 8 * (r >> 2) + 4 * hi + (r & 3); }

template <bool FULL>
__device__ __forceinline__ uint32_t survivors(const f32x16& acc, int sub_base, int n, int hi, float thr) {
  uint32_t m = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) m |= ((FULL || sub_of(sub_base, r, hi) < n) && acc[r] > thr ? 1u : 0u) << r;
  return m;
}

// Pass 2: offer one 32-sub-key tile (this lane: 16 sub-keys of token `tok`).
template <bool FULL>
__device__ __forceinline__ void offer_tile(const f32x16& acc, int sub_base, int n, int lane, int tok, int hi, int k,
                                           uint64_t* cand_wave, TokState& st) {
  uint32_t m = survivors<FULL>(acc, sub_base, n, hi, st.thr);
  if (__ballot(m != 0) == 0) return;
  int c = __popc(m);
  int co = __shfl_xor(c, 32, WAVE);
  uint64_t bal = __ballot(st.np + c + co > st.cap()) & 0xFFFFFFFFull;
  if (bal) {
    while (bal) {
      const int jj = __builtin_ctzll(bal);
      bal &= bal - 1;
      merge_token(cand_wave, jj, lane, tok, k, st);
    }
    m = survivors<FULL>(acc, sub_base, n, hi, st.thr);
    c = __popc(m);
    co = __shfl_xor(c, 32, WAVE);
  }
  int off = st.pbase() + st.np + (hi ? co : 0);
  uint64_t* b = cand_wave + tok * SLOTS;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (m & (1u << r)) b[off++] = make_key(acc[r], (uint32_t)sub_of(sub_base, r, hi));
  }
  st.np += c + co;
}

// k-th largest of the values v0, v1 held by all 64 lanes (ordered-float bits; 0 = absent):
// the largest x with #{v >= x} >= k, found bit by bit from the top with wave ballots.
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t v0, uint32_t v1, int k) {
  uint32_t prefix = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    const int cnt = __popcll(__ballot(v0 >= cand)) + __popcll(__ballot(v1 >= cand));
    if (cnt >= k) prefix = cand;
  }
  return prefix;
}

template <typename DT, int DH>
__global__ void __launch_bounds__(256, 2) score_topk_kernel(const DT* __restrict__ qhat, const DT* __restrict__ khat,
                                                            int64_t T, int H, int n, int k,
                                                            int32_t* __restrict__ half_idx,
                                                            float* __restrict__ half_score) {
  using M = Mma<DT, DH>;
  constexpr int RB = DH * M::EB;          // bytes per sub-key row
  constexpr int U16 = RB / 16;            // 16-byte units per row
  constexpr int UPT = CHUNK * U16 / 256;  // units per thread per chunk
  constexpr int MAXG = 128;               // group maxima per token kept by pass 1
  static_assert(UPT >= 1 && CHUNK * U16 % 256 == 0, "chunk must split evenly over 256 threads");
  static_assert(MAXG * 4 == SLOTS * 8, "pass-1 maxima reuse the candidate slots");

  __shared__ __attribute__((aligned(16))) uint8_t ks[CHUNK * RB];
  __shared__ uint64_t cand[TPB * SLOTS];

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
  const int swz_r = (lane & 31) % U16;
  const uint8_t* myrow = ks + (lane & 31) * RB;
  // stage chunk ch into LDS (the caller has prefetched it into `pre`), prefetch ch + 1, score it
  auto score_chunk = [&](int ch) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * 256;
      const int row = u / U16, col = u - row * U16;
      *(u32x4*)(ks + row * RB + ((col ^ (row % U16)) << 4)) = pre[i];
    }
    __syncthreads();
    if (ch + 1 < nch) fetch(ch + 1);
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < M::NK; ++kk) acc = M::mma(M::lds_k(myrow, swz_r, kk, hi), qf[kk], acc);
    return acc;
  };

  uint64_t* cand_wave = cand + wv * TPW * SLOTS;
  float* gmax_wave = (float*)cand_wave;  // pass 1: [token][MAXG] group maxima

  // ---- pass 1: the maximum score of each group of sub-keys, per token ------------------
  // The k-th largest of these maxima is a score that at least k sub-keys reach, so it
  // bounds the token's k-th best score from below.
  const int gsz = (nch + MAXG - 1) / MAXG;   // chunks per group
  const int ngroups = (nch + gsz - 1) / gsz;
  fetch(0);
  float gm = -__builtin_inff();
  for (int ch = 0; ch < nch; ++ch) {
    const f32x16 acc = score_chunk(ch);
    float m = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) m = sub_of(ch * CHUNK, r, hi) < n ? fmaxf(m, acc[r]) : m;
    m = fmaxf(m, __shfl_xor(m, 32, WAVE));
    gm = fmaxf(gm, m);
    if ((ch + 1) % gsz == 0 || ch + 1 == nch) {
      if (hi == 0) gmax_wave[tok * MAXG + ch / gsz] = gm;
      gm = -__builtin_inff();
    }
  }
  __builtin_amdgcn_wave_barrier();
  TokState st;
  st.nl = 0;
  st.np = 0;
  st.thr = -__builtin_inff();
  if (ngroups >= k) {
    for (int jj = 0; jj < TPW; ++jj) {
      const uint32_t v0 = lane < ngroups ? ord_score(gmax_wave[jj * MAXG + lane]) : 0u;
      const uint32_t v1 = lane + 64 < ngroups ? ord_score(gmax_wave[jj * MAXG + lane + 64]) : 0u;
      const uint32_t kth = wave_kth_largest(v0, v1, k);
      if (tok == jj) st.thr = float_below(score_of_ord(kth));
    }
  }
  __builtin_amdgcn_wave_barrier();

  // ---- pass 2: collect the sub-keys at or above the bound, keep the exact top-k -------
  fetch(0);
  for (int ch = 0; ch < nch; ++ch) {
    const f32x16 acc = score_chunk(ch);
    if ((ch + 1) * CHUNK <= n) offer_tile<true>(acc, ch * CHUNK, n, lane, tok, hi, k, cand_wave, st);
    else offer_tile<false>(acc, ch * CHUNK, n, lane, tok, hi, k, cand_wave, st);
  }

  // final merge of every token of this wave, then write its top-k
  for (int jj = 0; jj < TPW; ++jj) {
    merge_token(cand_wave, jj, lane, tok, k, st);
    const int64_t tj = tile * TPB + wv * TPW + jj;
    if (tj < T && lane < k) {
      const uint64_t key = cand_wave[jj * SLOTS + lane];
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
