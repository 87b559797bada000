// Sub-key scoring and the candidates of the per-half top-k.
//
// For each (token t, head h, half c), a "row": s[i] = <qhat_c[t, h], khat[h, c, i]> for
// all i < n_sub ("Memory Layers at Scale" digest, product-key search: a key is two
// sub-keys, so each half is scored against sqrt(N) sub-keys; "Memory inside the model"
// overview, how it works: each half is compared with its own list of half-keys and the
// best ones are kept).  The k best of every row, under (score desc, index asc), are
// chosen from the candidates written here by the combine kernel.
//
// Design for gfx950:
//  * The scores are a dense contraction (tokens x sub-keys x d_h) on the matrix cores:
//    v_mfma_f32_32x32x16_bf16 (bf16), v_mfma_f32_32x32x2f32 (fp32) or, for the fp8 bound
//    pass, v_mfma_scale_f32_32x32x64_f8f6f4, computing S^T = Khat * Qhat^T so that each
//    lane's 16 accumulators belong to ONE token.  A wave owns 64 tokens (two 32-token MFMA
//    columns), so every 16-byte LDS operand read feeds two MFMAs.  A block is 4 or 8 waves
//    = 256 or 512 tokens of one (h, c); 32-sub-key chunks reach a double-buffered,
//    XOR-swizzled LDS tile shared by the block's waves by direct buffer->LDS loads, the
//    next chunks while the current ones are scored.  Pass 2 also keeps a small per-lane row
//    of scores in LDS for its appends.
//  * The scores are never written out; selection takes two passes:
//      pass 1 writes, per row, the maximum score of every group of G consecutive
//             sub-keys (G in {8, 16, 32, 64, ...}, the smallest giving <= 128 groups),
//             then theta in its tail: the k-th largest group maximum, rounded down to its
//             top 16 bits: at least k sub-keys reach it, so it bounds the row's k-th best
//             score from below (with split sub-key ranges theta_kernel forms it instead).
//             With the fp8 bound the maxima are of fp8 scores and theta is lowered by a
//             margin: an estimate, which the counts of pass 2 check;
//      pass 2 recomputes the scores exactly and writes every sub-key scoring at or above
//             the bound as a 64-bit key to the row's candidate list (cand_slots(k) slots,
//             half per lane).  With random-like data and k = 32 about 37 of 4,096 per row
//             (48 with the fp8 bound's margin).
//    A lane's count may exceed its half of the slots (structured data), or the two halves
//    hold fewer than k (an fp8 estimate set too high); that row is then scored exhaustively
//    by the overflow kernel before the combine kernel reads it.
//  * With fewer than 2k groups (k + 32 for k > 32: few sub-keys for the k asked for) the
//    bound prunes little and most rows would overflow: every row is then scored
//    exhaustively, one wave per row, instead of the two passes.
//  * Keys are 64-bit (ordered score << 32 | ~index): ties resolve to the lower index
//    and every key is distinct.
//  * Blocks are numbered so that block b works on pair (h, c) = b mod 2H; blocks are
//    dealt round-robin to the 8 XCDs, so with 2H dividing 8 each XCD only ever reads
//    one pair's sub-keys, which stay resident in that XCD's L2.
//  * A batch too small to give every CU a block splits the sub-keys into ranges of whole
//    chunks, one block per (tile, range, pair): pass 1 writes each range's group maxima,
//    and pass 2's ranges share a row's candidate list through atomic counts (cleared by
//    the first range's pass 1 blocks), each lane staging up to 9-16 candidates in LDS
//    and taking their slots with one atomic.
#include "kernels.hpp"

namespace pkm {

namespace {

// A wave scores FR token fragments of 32 (one 32-token MFMA column each): FR = 2 (64
// tokens per wave) reuses every LDS operand read for two MFMAs; FR = 1 serves batches too
// small to give every CU eight 64-token waves per pair.
constexpr int CHUNK = 32;       // sub-keys per LDS chunk (one 32-row MFMA tile)
// chunks loaded per barrier: 8-wave blocks (one per CU, LDS to spare) take two chunks
// between barriers, which halves the barriers and the skew every one of them absorbs
// (fp8 chunks, half the bytes and half the MFMA time of bf16 ones, go four to a barrier)
constexpr int chunks_per_barrier(int nw, int eb = 2) { return nw == 8 ? (eb == 1 ? 4 : 2) : 1; }

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

// fp8 (OCP e4m3), the bound pass of bf16 workloads: A = 32 sub-keys x 64 dims (lane: row l%32,
// 32 consecutive dims from (l/32)*32 of each 64-dim k-step), B = 64 dims x 32 tokens, the same
// dims per lane; v_mfma_f32_32x32x64_f8f6f4 without scaling, the 32 x 32 fp32 result laid out
// as for bf16.
template <int DH>
struct Mma<uint8_t, DH> {
  static constexpr int KSTEP = 64;
  static constexpr int NK = DH / KSTEP;
  static constexpr int EB = 1;
  typedef i32x8 frag;
  __device__ static frag load_q(const uint8_t* q, int kk, int hi) { return *(const i32x8*)(q + kk * KSTEP + hi * 32); }
  // 16-byte units 4 kk + 2 hi and the next one of the lane's row
  __device__ static frag lds_k(const uint8_t* row, int swz, int kk, int hi) {
    const u32x4 lo = *(const u32x4*)(row + (((4 * kk + 2 * hi) ^ swz) << 4));
    const u32x4 up = *(const u32x4*)(row + (((4 * kk + 2 * hi + 1) ^ swz) << 4));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
  }
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

__device__ __forceinline__ float load_elem_f32(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_elem_f32(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }

__device__ __forceinline__ int sub_of(int sub_base, int r, int hi) { return sub_base + 8 * (r >> 2) + 4 * hi + (r & 3); }

// The shared MFMA sweep over all sub-keys of one pair for the block's NW * FR * 32 tokens.
// `on_tile(ch, acc)` receives, per 32-sub-key chunk, the scores of this lane's FR tokens
// (acc[g]: token 32 g + lane%32 of the wave).
//
// NW = 4: one wave per SIMD per block, two blocks per CU.  Both blocks start together and
// do the same work, so their two waves on a SIMD run in step: both issue MFMAs, then both
// run the selection on the VALU, then both wait at the barrier, and the matrix core idles
// through the second half.  NW = 8: one block of 8 waves per CU, waves w and w + 4 sharing
// a SIMD; the second group takes each chunk's scores one chunk late (its selection of
// chunk ch - 1 runs right after the barrier, beside the first group's MFMAs of chunk ch,
// and its MFMAs of chunk ch beside the first group's selection), which keeps the matrix
// core fed through both halves.  The accumulators live across the barrier for that.
template <typename DT, int DH, int NW, int FR, bool TWO, typename F>
__device__ __forceinline__ void sweep(const DT* __restrict__ qhat, const DT* __restrict__ khat, int64_t T, int H, int n,
                                      int pair, int64_t tile, int c0, int c1, uint8_t* ka, uint8_t* kb,
                                      F&& on_tile) {
  using M = Mma<DT, DH>;
  constexpr int RB = DH * M::EB;          // bytes per sub-key row
  constexpr int U16 = RB / 16;            // 16-byte units per row

  const int h = pair >> 1, c = pair & 1;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6), hi = lane >> 5;

  typename M::frag qf[FR][M::NK];
#pragma unroll
  for (int g = 0; g < FR; ++g) {
    const int64_t t = tile * (32 * FR * NW) + wv * (32 * FR) + g * 32 + (lane & 31);
    const DT* qrow = qhat + ((t * H + h) * 2 + c) * (int64_t)DH;
#pragma unroll
    for (int kk = 0; kk < M::NK; ++kk) qf[g][kk] = t < T ? M::load_q(qrow, kk, hi) : typename M::frag{};
  }

  const uint8_t* kbase = (const uint8_t*)(khat + (size_t)pair * n * DH);
  // Chunk ch goes to an LDS buffer by direct global->LDS loads: wave wv's i-th load fills
  // the 64 consecutive 16-byte units starting at unit (wv * DPW + i) * 64, and each lane
  // fetches the global unit that belongs at its LDS unit under the XOR swizzle.  Rows past
  // n_sub load row 0 instead (in bounds); their scores are masked by every consumer.
  // The loads are buffer loads (a descriptor over this pair's n_sub * RB bytes) rather than
  // global ones: the compiler counts a global load into LDS as both a memory and an LDS
  // access, and then waits for every LDS read in flight (lgkmcnt(0)) before each MFMA
  // operand instead of only the one it needs, which exposed the LDS latency four times
  // per chunk.
  constexpr int DPW = CHUNK * U16 / 64 / NW;  // loads per wave per chunk
  static_assert(DPW >= 1 && CHUNK * U16 % (64 * NW) == 0, "chunk must split evenly over the waves");
  const __amdgpu_buffer_rsrc_t krsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, n * RB, 0x00020000);  // raw, 32-bit dwords
  auto fetch = [&](int ch, uint8_t* dst) {
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int p = (wv * DPW + i) * 64 + lane;          // LDS unit this lane fills
      const int row = p / U16, col = (p % U16) ^ (row % U16);
      int sub = ch * CHUNK + row;
      sub = sub < n ? sub : 0;
      // a 32-bit offset from the wave-uniform base (one pair's sub-keys: n_sub * RB < 2^32
      // bytes) keeps one VGPR per address; 64-bit per-lane addresses made pass 2 spill
      // them, and every reload from scratch waited for all loads in flight
      const uint32_t off = (uint32_t)sub * RB + (uint32_t)col * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          krsrc, (void __attribute__((address_space(3)))*)(dst + (wv * DPW + i) * 64 * 16), 16, off, 0, 0, 0);
    }
  };
  const int swz = (lane & 31) % U16;

  // The block sweeps chunks [c0, c1) in groups of SC chunks, one barrier per group.  The
  // groups alternate between two LDS buffers (ka, kb: SC chunks each): a group is scored
  // from one while the next group's chunks load into the other.  TWO: the buffers are two
  // LDS arrays and the group's code is inlined once for each, so that the compiler knows
  // that the MFMA operand reads cannot touch the buffer the loads in flight are filling;
  // pass 2 needs it, where the compiler otherwise waited for those loads (and for the
  // candidate stores, which share their counter) before every chunk.  Otherwise (pass 1,
  // whose registers do not allow two copies) kb follows ka in one array and one loop
  // indexes the 2 SC chunk buffers.
  constexpr int SC = chunks_per_barrier(NW, M::EB);
  constexpr int CB = CHUNK * RB;  // bytes per chunk buffer
  // the lagging group (wave-uniform)
  const bool lag = NW == 8 && wv >= 4;
  f32x16 acc[FR];
  // bf16 and fp8: the LDS operands run PD k-steps ahead of the MFMAs; the scheduling groups
  // below keep the compiler from pulling the reads back next to their use (it otherwise
  // waits for the LDS every two k-steps).  An fp8 operand is two LDS reads.  (Reading the
  // next fp8 chunk's operands before the current chunk's selection was 5-10 us slower.)
  // (fp32 keeps the plain loop: with one-register operands the groups only lengthen live
  // ranges and cause spills.)
  constexpr int PD = 4 < M::NK ? 4 : M::NK;
  constexpr int RD = M::EB == 1 ? 2 : 1;  // LDS reads per operand
  // the scores of the chunk at this lane's row `row`
  auto score_chunk = [&](const uint8_t* row) {
#pragma unroll
    for (int g = 0; g < FR; ++g) acc[g] = f32x16{};
    if constexpr (M::EB != 4) {
      typename M::frag a[M::NK];
#pragma unroll
      for (int kk = 0; kk < PD; ++kk) a[kk] = M::lds_k(row, swz, kk, hi);
#pragma unroll
      for (int kk = 0; kk < M::NK; ++kk) {
        if (kk + PD < M::NK) a[kk + PD] = M::lds_k(row, swz, kk + PD, hi);
#pragma unroll
        for (int g = 0; g < FR; ++g) acc[g] = M::mma(a[kk], qf[g][kk], acc[g]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, RD * PD, 0);  // DS reads
#pragma unroll
      for (int kk = 0; kk < M::NK; ++kk) {
        if (kk + PD < M::NK) __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, FR, 0);     // MFMAs
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < M::NK; ++kk) {
        const typename M::frag b = M::lds_k(row, swz, kk, hi);
#pragma unroll
        for (int g = 0; g < FR; ++g) acc[g] = M::mma(b, qf[g][kk], acc[g]);
      }
    }
  };
#pragma unroll
  for (int j = 0; j < SC; ++j)
    if (c0 + j < c1) fetch(c0 + j, ka + j * CB);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads have landed in LDS
  __syncthreads();
  if constexpr (TWO) {
    auto group = [&](int g0, const uint8_t* cur, uint8_t* nxt) {
#pragma unroll
      for (int j = 0; j < SC; ++j)
        if (g0 + SC + j < c1) fetch(g0 + SC + j, nxt + j * CB);
      const uint8_t* rows = cur + (lane & 31) * RB;  // this lane's row of chunk 0 of the group
      for (int j = 0; j < SC && g0 + j < c1; ++j) {
        const int ch = g0 + j;
        if (lag && ch > c0) on_tile(ch - 1, (const f32x16*)acc);
        score_chunk(rows + j * CB);
        if (!lag) on_tile(ch, (const f32x16*)acc);
      }
      // this group's reads are done and the next group's chunks have landed
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
    };
    for (int g0 = c0; g0 < c1; g0 += 2 * SC) {
      group(g0, ka, kb);
      if (g0 + SC < c1) group(g0 + SC, kb, ka);
    }
  } else {
    // the chunk at position lc = ch - c0 lives in buffer lc % (2 SC) of ka (kb = ka + SC CB)
    const uint8_t* rows = ka + (lane & 31) * RB;
    for (int ch = c0; ch < c1; ++ch) {
      const int lc = ch - c0;
      const int buf = lc % (2 * SC);
      // the other SC buffers were last read before the barrier that ended the previous group
      if (lc % SC == 0) {
#pragma unroll
        for (int j = 0; j < SC; ++j)
          if (ch + SC + j < c1) fetch(ch + SC + j, ka + ((lc + SC + j) % (2 * SC)) * CB);
      }
      if (lag && lc > 0) on_tile(ch - 1, (const f32x16*)acc);
      score_chunk(rows + buf * CB);
      if (!lag) on_tile(ch, (const f32x16*)acc);
      if (lc % SC == SC - 1 || ch + 1 == c1) {  // the group's last chunk
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
      }
    }
  }
  if (lag) on_tile(c1 - 1, (const f32x16*)acc);
}

// Block b: pair (h, c) = b mod 2H (so each XCD only reads one pair's sub-keys), then the
// split of the sub-key chunks, then the token tile.  A batch too small to give every CU a
// block sweeps the sub-keys in `splits` ranges of `cps` chunks, one block each.
struct BlockPos {
  int pair, c0, c1, split;
  int64_t tile;
};
__device__ __forceinline__ BlockPos block_pos(int H, int n, int splits, int cps) {
  const int pairs = 2 * H;
  const int64_t rest = blockIdx.x / pairs;
  BlockPos p;
  p.pair = blockIdx.x % pairs;
  p.split = (int)(rest % splits);
  p.tile = rest / splits;
  const int nch = (n + CHUNK - 1) / CHUNK;
  p.c0 = p.split * cps;
  p.c1 = p.c0 + cps < nch ? p.c0 + cps : nch;
  return p;
}

// The bound theta of the selection (see theta_kernel): its ordered key keeps the top THETA_BITS
// bits.  ThetaArgs: where pass 1 writes it itself (theta non-NULL) and, for the fp8 bound, the
// norms its margin scales with.
constexpr int THETA_BITS = 16;
struct ThetaArgs {
  float* theta = nullptr;
  int k = 0;
  const float* qn = nullptr;
  const float* kmax = nullptr;
  float eta = 0.f;
};

// Max over the 16 scores of one lane, or only over those of sub-keys < n.
template <bool FULL>
__device__ __forceinline__ float lane_max(const f32x16& a, int sub_base, int n, int hi, int r0, int r1) {
  float m = -__builtin_inff();
#pragma unroll
  for (int r = r0; r < r1; ++r) m = (FULL || sub_of(sub_base, r, hi) < n) ? fmaxf(m, a[r]) : m;
  return m;
}

// Pass 1: per row, the maximum of every group of G = 8 << GS sub-keys.  The maxima of
// NB consecutive groups are collected in registers (a shift register) and written as
// 16-byte stores, so that few stores are in flight when a chunk waits for its loads
// (NB = 4 with 8-wave blocks, whose lagging group holds its accumulators across the
// barrier: 8 spilled there).
template <typename DT, int DH, int GS, int NW, int FR>
__global__ void __launch_bounds__(64 * NW, 8 / NW) pass1_kernel(const DT* __restrict__ qhat, const DT* __restrict__ khat,
                                                       int64_t T, int H, int n, int splits, int cps,
                                                       float* __restrict__ gmax, int32_t* __restrict__ zero_count,
                                                       ThetaArgs ta) {
  constexpr int RB = DH * Mma<DT, DH>::EB;
  constexpr int GPC = GS <= 2 ? (4 >> GS) : 1;        // groups finished per chunk (or per span)
  constexpr int SPAN = GS <= 2 ? 1 : (1 << (GS - 2)); // chunks per group when a group spans chunks
  constexpr int KB = chunks_per_barrier(NW, Mma<DT, DH>::EB) * CHUNK * RB;  // bytes per buffer
  __shared__ __attribute__((aligned(16))) uint8_t ks[2 * KB];
  const BlockPos bp = block_pos(H, n, splits, cps);
  const int pair = bp.pair;
  const int64_t tile = bp.tile;
  const int h = pair >> 1, c = pair & 1;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), hi = lane >> 5;
  constexpr int NB = NW == 8 ? 4 : 8;
  float run[FR];
  float buf[FR][NB];
  int nbuf = 0;  // groups in buf (wave-uniform)
#pragma unroll
  for (int g = 0; g < FR; ++g) {
    run[g] = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < NB; ++j) buf[g][j] = 0.f;
  }
  float* gm[FR];
  bool live[FR];
#pragma unroll
  for (int g = 0; g < FR; ++g) {
    const int64_t t = tile * (32 * FR * NW) + wv * (32 * FR) + g * 32 + (lane & 31);
    live[g] = t < T;  // both lanes of a row store its group maxima (the same values)
    const int64_t r2 = (t * H + h) * 2 + c;
    gm[g] = gmax + r2 * (int64_t)MAX_GROUPS;
    // with split sub-key ranges pass 2 counts every row's candidates with atomics: the
    // first split clears the counts (both lane halves of the row)
    if (zero_count && bp.split == 0 && t < T) zero_count[r2 * 2 + hi] = 0;
  }
  // groups written: the split starts at a group boundary that is a multiple of NB groups
  int done = GS <= 2 ? bp.c0 * GPC : bp.c0 / SPAN;
  auto push = [&](const float* m) {  // one finished group per token of this lane
#pragma unroll
    for (int g = 0; g < FR; ++g) {
#pragma unroll
      for (int j = 0; j < NB - 1; ++j) buf[g][j] = buf[g][j + 1];
      buf[g][NB - 1] = m[g];
    }
    // shift register: the newest is buf[NB - 1]; after NB pushes buf[0] is the oldest
    if (++nbuf == NB) {
#pragma unroll
      for (int g = 0; g < FR; ++g) {
        if (!live[g]) continue;
#pragma unroll
        for (int j = 0; j < NB; j += 4)
          *(f32x4*)(gm[g] + done + j) = f32x4{buf[g][j], buf[g][j + 1], buf[g][j + 2], buf[g][j + 3]};
      }
      done += NB;
      nbuf = 0;
    }
  };
  sweep<DT, DH, NW, FR, false>(qhat, khat, T, H, n, pair, tile, bp.c0, bp.c1, ks, ks + KB, [&](int ch, const f32x16* acc) {
    const bool full = (ch + 1) * CHUNK <= n;
    float mg[FR][GPC];
#pragma unroll
    for (int g = 0; g < FR; ++g) {
      // a group of 8 << GS sub-keys inside the chunk covers rows [4j, 4j + 4 << GS) of both lanes
#pragma unroll
      for (int j = 0; j < GPC; ++j) {
        constexpr int RW = GS <= 2 ? (4 << GS) : 16;
        const float m = full ? lane_max<true>(acc[g], ch * CHUNK, n, hi, j * RW, j * RW + RW)
                             : lane_max<false>(acc[g], ch * CHUNK, n, hi, j * RW, j * RW + RW);
        mg[g][j] = max_xor32(m);
      }
    }
    if (GS <= 2) {
#pragma unroll
      for (int j = 0; j < GPC; ++j) {
        if (ch * CHUNK + j * (8 << GS) < n) {
          float m[FR];
#pragma unroll
          for (int g = 0; g < FR; ++g) m[g] = mg[g][j];
          push(m);
        }
      }
    } else {
#pragma unroll
      for (int g = 0; g < FR; ++g) run[g] = fmaxf(run[g], mg[g][0]);
      if (((ch + 1) & (SPAN - 1)) == 0 || (ch + 1) * CHUNK >= n) {
        push(run);
#pragma unroll
        for (int g = 0; g < FR; ++g) run[g] = -__builtin_inff();
      }
    }
  });
  // the last < NB groups: buf[NB - nbuf .. NB - 1] hold groups done .. done + nbuf - 1
#pragma unroll
  for (int g = 0; g < FR; ++g) {
    if (!live[g]) continue;
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (i < nbuf) gm[g][done + i] = buf[g][NB - nbuf + i];
  }
  // theta of every row of the block (sub-keys not split: the block has all its group maxima),
  // instead of the theta kernel: the row's two lanes take 64 of its 128 slots each, 16-byte
  // pieces of their own stores, and run the descent of theta_kernel with their counts summed.
  // Every group maximum of a row lies in [vmin, vmax], so theta shares their leading bits:
  // the descent starts at the highest bit where the two differ (the wave's highest, found
  // with five ballots, so that the steps stay uniform; a row whose bit is already settled
  // keeps its prefix at that step).  That skips the sign and most exponent bits, about a
  // third of the steps, with the result of the full descent.
  if (ta.theta) {
    const int ngroups = (n + (8 << GS) - 1) >> (3 + GS);
#pragma unroll
    for (int g = 0; g < FR; ++g) {
      uint32_t v[MAX_GROUPS / 2];
      uint32_t vmin = 0xFFFFFFFFu, vmax = 0u;
#pragma unroll
      for (int p = 0; p < MAX_GROUPS / 8; ++p) {  // piece 2 p + hi: groups 8 p + 4 hi .. + 3
        const int g0 = 8 * p + 4 * hi;
        const f32x4 x = live[g] && g0 < ngroups ? *(const f32x4*)(gm[g] + g0) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = live[g] && g0 + e < ngroups;
          const uint32_t o = ord_score(x[e]);
          v[4 * p + e] = ok ? o : 0u;
          vmin = ok && o < vmin ? o : vmin;
          vmax = ok && o > vmax ? o : vmax;
        }
      }
      {  // the row's two lanes
        const auto a = __builtin_amdgcn_permlane32_swap(vmin, vmin, false, false);
        const auto b = __builtin_amdgcn_permlane32_swap(vmax, vmax, false, false);
        vmin = a[0] < a[1] ? a[0] : a[1];
        vmax = b[0] > b[1] ? b[0] : b[1];
      }
      const uint32_t d = vmin ^ vmax;
      const int hb = d ? 31 - __builtin_clz(d) : 0;
      uint32_t prefix = vmax & ~((2u << hb) - 1u);  // the bits above hb (none for hb = 31)
      int top = 0;
#pragma unroll
      for (int b5 = 4; b5 >= 0; --b5)
        if (__ballot(hb >= (top | (1 << b5)))) top |= 1 << b5;
#pragma unroll
      for (int bit = 31; bit >= 32 - THETA_BITS; --bit) {
        if (bit > top) continue;
        const uint32_t cand = prefix | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < MAX_GROUPS / 2; ++j) cnt += v[j] >= cand ? 1 : 0;
        cnt = add_xor32(cnt);
        if (cnt >= ta.k) prefix = cand;
      }
      prefix &= ~((1u << (32 - THETA_BITS)) - 1u);
      const int64_t t = tile * (32 * FR * NW) + wv * (32 * FR) + g * 32 + (lane & 31);
      if (hi == 0 && t < T) {
        const int64_t r2 = (t * H + h) * 2 + c;
        float th = ngroups < ta.k ? -__builtin_inff() : score_of_ord(prefix);
        if (ta.qn) th -= ta.eta * ta.qn[r2] * ta.kmax[pair];
        ta.theta[r2] = th;
      }
    }
  }
}

// theta: per row a lower bound of the k-th largest of its group maxima (-inf if there are
// fewer than k).  Any value at or below that k-th largest bounds the row's k-th score from
// below, so the descent stops after the top THETA_BITS bits of the ordered key (sign,
// exponent and 7 mantissa bits: within 2^-7 of the k-th group maximum, which adds about one
// candidate per row) and takes the prefix with zero low bits.  The kernel is bound by the
// scalar unit (popcounts, adds and compares per bit): 16 bits instead of 32 took it from
// 54 to 34 us at 131,072 rows.
// Keys strictly above a bound that is below the k-th group maximum already number at least
// k, so the cap on keys equal to the bound (pass 2 over split sub-key ranges) drops none that
// matter.
// With group maxima of fp8 scores (qn != NULL) the k-th largest is only an estimate: the bound
// is lowered by eta * |q half| * max |sub-key| of the pair, a few standard deviations of the
// fp8 rounding error of a score.  Pass 2 then still counts the exact scores at or above it, and
// a row left with fewer than k is scored exhaustively, so the bound decides only the work.
__global__ void __launch_bounds__(256) theta_kernel(const float* __restrict__ gmax, int64_t rows, int ngroups, int k,
                                                    float* __restrict__ theta, const float* __restrict__ qn,
                                                    const float* __restrict__ kmax, int pairs, float eta) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  if (ngroups < k) {
    if (lane == 0) theta[row] = -__builtin_inff();
    return;
  }
  const float* gm = gmax + row * MAX_GROUPS;
  const uint32_t v0 = lane < ngroups ? ord_score(gm[lane]) : 0u;
  const uint32_t v1 = lane + 64 < ngroups ? ord_score(gm[lane + 64]) : 0u;
  // largest x (low 32 - THETA_BITS bits zero) with #{v >= x} >= k, bit by bit from the top
  uint32_t prefix = 0;
#pragma unroll
  for (int bit = 31; bit >= 32 - THETA_BITS; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    const int cnt = __popcll(__ballot(v0 >= cand)) + __popcll(__ballot(v1 >= cand));
    if (cnt >= k) prefix = cand;
  }
  if (lane == 0) theta[row] = qn ? score_of_ord(prefix) - eta * qn[row] * kmax[row % pairs] : score_of_ord(prefix);
}

// Pass 2: write the candidates of every row (keys at or above theta; with split sub-key
// ranges only the first k per lane of those equal to theta).  Each of a token's two lanes
// owns `half` of the row's 2 * half slots and counts its own candidates.
template <typename DT, int DH, int NW, int FR, bool SPLIT>
__global__ void __launch_bounds__(64 * NW, 8 / NW) pass2_kernel(const DT* __restrict__ qhat, const DT* __restrict__ khat,
                                                       int64_t T, int H, int n, int k, int splits, int cps,
                                                       const float* __restrict__ theta, uint64_t* __restrict__ cand,
                                                       int32_t* __restrict__ count, int half) {
  constexpr int RB = DH * Mma<DT, DH>::EB;
  // SROW floats per lane: the lane's 16 FR scores of the chunk, read back by position for
  // the appends (36 or 20, not 32 or 16: 16-byte stores of 16 consecutive lanes then hit
  // distinct banks)
  constexpr int SROW = 16 * FR + 4;
  // split sub-key ranges: a lane keeps up to STASH of its candidates in LDS and publishes
  // them with one atomic count per stash (an atomic per candidate, waited for before its
  // store, cost 15-17% of the four scoring kernels at 256-4,096 tokens); STASH fills what
  // the block's share of the CU's 160 KiB of LDS leaves, up to 16
  constexpr int LDS_USED = 2 * chunks_per_barrier(NW) * CHUNK * RB + NW * 64 * SROW * 4;
  constexpr int STASH_FIT = (160 * 1024 / (8 / NW) - LDS_USED) / (FR * NW * 64 * 8);
  constexpr int STASH = SPLIT ? (STASH_FIT < 16 ? STASH_FIT : 16) : 1;
  static_assert(STASH >= 1, "no LDS left for the candidate stash");
  __shared__ __attribute__((aligned(16))) uint8_t ka[chunks_per_barrier(NW) * CHUNK * RB];
  __shared__ __attribute__((aligned(16))) uint8_t kb[chunks_per_barrier(NW) * CHUNK * RB];
  __shared__ __attribute__((aligned(16))) float stage[NW * 64 * SROW];
  __shared__ uint64_t stash[SPLIT ? STASH * FR * NW * 64 : 1];
  const BlockPos bp = block_pos(H, n, splits, cps);
  const int pair = bp.pair;
  const int64_t tile = bp.tile;
  const int h = pair >> 1, c = pair & 1;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), hi = lane >> 5;
  float thr[FR];
  int cnt[FR], eq[FR];
  uint64_t* dst[FR];
  int64_t row[FR];
#pragma unroll
  for (int g = 0; g < FR; ++g) {
    cnt[g] = eq[g] = 0;
    const int64_t t = tile * (32 * FR * NW) + wv * (32 * FR) + g * 32 + (lane & 31);
    row[g] = (t * H + h) * 2 + c;
    thr[g] = t < T ? theta[row[g]] : __builtin_inff();
    dst[g] = cand + row[g] * (2 * half) + hi * half;
  }
  // thz: the bound with a zero bound taken as -0, so that the sign of (score - thz) is
  // set exactly when score < bound, -0 scores included (x - x is +0; finite values)
  float thz[FR];
#pragma unroll
  for (int g = 0; g < FR; ++g) thz[g] = thr[g] == 0.f ? -0.f : thr[g];
  float* my = stage + (wv * 64 + lane) * SROW;
  // stash slot i of fragment g: consecutive lanes at consecutive words
  auto stash_at = [&](int g, int i) -> uint64_t& { return stash[((i * FR + g) * NW + wv) * 64 + lane]; };
  // the row's lane-half list gets nst more keys: slots by one atomic count (a count beyond
  // `half` sends the row to the overflow pass, as a full list does)
  auto publish = [&](int g, int nst) {
    const int base = atomicAdd(count + (g ? row[FR - 1] : row[0]) * 2 + hi, nst);
    uint64_t* d = g ? dst[FR - 1] : dst[0];
    for (int i = 0; i < nst; ++i)
      if (base + i < half) d[base + i] = stash_at(g, i);
  };
  sweep<DT, DH, NW, FR, true>(qhat, khat, T, H, n, pair, tile, bp.c0, bp.c1, ka, kb, [&](int ch, const f32x16* acc) {
    const bool full = (ch + 1) * CHUNK <= n;
    // bit 16 g + r: score r of token fragment g reaches the bound.  The sign bits of the
    // differences are shifted in with v_alignbit: two VALU ops per score and no lane
    // masks (a compare and select per score costs twice that, with a wait state after
    // every compare).
    uint32_t m = 0;
#pragma unroll
    for (int g = 0; g < FR; ++g) {
      uint32_t miss = 0;
#pragma unroll
      for (int r = 15; r >= 0; --r) miss = __builtin_amdgcn_alignbit(miss, __float_as_uint(acc[g][r] - thz[g]), 31);
      m |= (~miss & 0xFFFFu) << (16 * g);
    }
    if (!full) {  // the last chunk: only sub-keys < n exist
      const int nv = n - ch * CHUNK;
      uint32_t valid = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) valid |= (8 * (r >> 2) + 4 * hi + (r & 3) < nv ? 1u : 0u) << r;
      m &= FR == 2 ? valid * 0x10001u : valid;
    }
    // the appends loop over the set bits only (both fragments in one loop), so the wave
    // runs as many rounds as its busiest lane has candidates in this chunk; a hit's score
    // comes back from the lane's own LDS row (a select over 16 registers by a per-lane
    // position cost 30 VALU ops per round)
    if (m) {
#pragma unroll
      for (int g = 0; g < FR; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *(f32x4*)(my + 16 * g + 4 * j) = f32x4{acc[g][4 * j], acc[g][4 * j + 1], acc[g][4 * j + 2], acc[g][4 * j + 3]};
    }
    if constexpr (SPLIT) {  // split sub-key ranges share the row's lane-half list
      while (m) {
        const int b = __builtin_ctz(m);  // fragment 0 first, ascending positions: the order of a scan
        m &= m - 1;
        const int g = b >> 4, r = b & 15;
        const float s = my[b];
        const int sub = sub_of(ch * CHUNK, r, hi);
        int cn = g ? cnt[FR - 1] : cnt[0];
        int e = g ? eq[FR - 1] : eq[0];
        bool take = true;
        if (s == (g ? thr[FR - 1] : thr[0])) take = e++ < k;  // exact ties with the bound: the first k suffice
        if (take) {
          if (cn == STASH) {
            publish(g, cn);
            cn = 0;
          }
          stash_at(g, cn) = make_key(s, (uint32_t)sub);
          ++cn;
        }
        if (g) {
          cnt[FR - 1] = cn;
          eq[FR - 1] = e;
        } else {
          cnt[0] = cn;
          eq[0] = e;
        }
      }
    } else {
      // The score of the lane's next hit is read from LDS before the current hit's key is
      // built, so that part of the read's latency overlaps that work.  The rounds have no
      // branches: a full list takes further keys in its last slot
      // (the row then goes to the overflow pass, which rewrites its list), and keys equal to
      // the bound are all taken (capping them only spares the overflow pass on structured
      // data, and cost a compare and two branches a round).
      int b = m ? __builtin_ctz(m) : 0;  // fragment 0 first, ascending positions: the order of a scan
      float s = my[b];
      while (m) {
        const int bh = b;
        const float sh = s;
        m &= m - 1;
        b = m ? __builtin_ctz(m) : 0;
        s = my[b];
        const int g = bh >> 4, r = bh & 15;
        const uint64_t key = make_key(sh, (uint32_t)sub_of(ch * CHUNK, r, hi));
        const int cn = g ? cnt[FR - 1] : cnt[0];
        (g ? dst[FR - 1] : dst[0])[cn < half ? cn : half - 1] = key;
        cnt[0] += g ? 0 : 1;
        if constexpr (FR == 2) cnt[1] += g;
      }
    }
  });
  if constexpr (SPLIT) {  // what is left in the stashes (rows past T have none)
#pragma unroll
    for (int g = 0; g < FR; ++g)
      if (cnt[g] > 0) publish(g, cnt[g]);
  } else {
#pragma unroll
    for (int g = 0; g < FR; ++g) {
      const int64_t t = tile * (32 * FR * NW) + wv * (32 * FR) + g * 32 + (lane & 31);
      if (t < T) count[row[g] * 2 + hi] = cnt[g];
    }
  }
}

// The exact top-k of one row (t, h, c) by exhaustive scoring in plain fp32 FMAs (d in
// ascending order): each lane keeps the best LK >= k keys of its share of the sub-keys in
// registers, the 64 lane lists are merged by k rounds of a wave-wide maximum, and the
// row's candidate list (cs slots) becomes exactly its top-k (count k in the first lane
// half, 0 in the second).  qs: this wave's LDS row of DH floats.
template <typename DT, int DH, int LK>
__device__ void exhaustive_row(const DT* __restrict__ qhat, const DT* __restrict__ khat, int64_t r2, int H, int n,
                               int k, uint64_t* __restrict__ cand, int cs, int32_t* __restrict__ count, float* qs,
                               int lane) {
  constexpr int VE = 16 / (int)sizeof(DT);  // elements per 16-byte load
  const int pair = (int)(r2 % (2 * H));
  const DT* q = qhat + r2 * DH;
  for (int d = lane; d < DH; d += 64) qs[d] = load_elem_f32(q, d);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  uint64_t L[LK];
#pragma unroll
  for (int j = 0; j < LK; ++j) L[j] = 0ull;
  const DT* kb = khat + (size_t)pair * n * DH;
  for (int i = lane; i < n; i += 64) {
    const u32x4* kr = (const u32x4*)(kb + (size_t)i * DH);
    float s = 0.f;
#pragma unroll 4
    for (int v = 0; v < DH / VE; ++v) {
      const u32x4 x = kr[v];
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        float kv;
        if constexpr (sizeof(DT) == 2) kv = (e & 1) ? bf16_hi(x[e >> 1]) : bf16_lo(x[e >> 1]);
        else kv = __uint_as_float(x[e]);
        s = __builtin_fmaf(qs[v * VE + e], kv, s);
      }
    }
    uint64_t key = make_key(s, (uint32_t)i);
    if (key > L[LK - 1]) {
#pragma unroll
      for (int j = 0; j < LK; ++j) {
        const uint64_t lo = key > L[j] ? L[j] : key;
        L[j] = key > L[j] ? key : L[j];
        key = lo;
      }
    }
  }
  for (int j = 0; j < k; ++j) {
    const uint64_t win = wave_max_u64(L[0]);
    if (L[0] == win) {
#pragma unroll
      for (int i = 0; i < LK - 1; ++i) L[i] = L[i + 1];
      L[LK - 1] = 0ull;
    }
    if (lane == 0) cand[r2 * cs + j] = win;
  }
  if (lane == 0) {
    count[2 * r2] = k;
    count[2 * r2 + 1] = 0;
  }
  __builtin_amdgcn_wave_barrier();
}

// Rows whose candidates overflowed (more than cs / 2 in either lane's half: structured
// data with many sub-keys above the bound), or, under an estimated bound, that hold fewer
// than k, are scored again exhaustively.  A persistent grid scans the counts; with neither
// it only reads them.
template <typename DT, int DH, int LK>
__global__ void __launch_bounds__(256) overflow_kernel(const DT* __restrict__ qhat, const DT* __restrict__ khat,
                                                       int64_t rows2, int H, int n, int k, uint64_t* __restrict__ cand,
                                                       int cs, int32_t* __restrict__ count) {
  __shared__ float qs[4][DH];
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t waves = (int64_t)gridDim.x * 4;
  for (int64_t base = ((int64_t)blockIdx.x * 4 + wv) * 64; base < rows2; base += waves * 64) {
    const int64_t r = base + lane;
    uint64_t over = __ballot(r < rows2 && (count[2 * r] > cs / 2 || count[2 * r + 1] > cs / 2 ||
                                           count[2 * r] + count[2 * r + 1] < k));
    while (over) {
      const int64_t r2 = base + __builtin_ctzll(over);
      over &= over - 1;
      exhaustive_row<DT, DH, LK>(qhat, khat, r2, H, n, k, cand, cs, count, qs[wv], lane);
    }
  }
}

// Few sub-keys per row (fewer than 2k groups, so the group-maximum bound prunes little and
// most rows would overflow): every row exhaustively, one wave per row.
template <typename DT, int DH, int LK>
__global__ void __launch_bounds__(256) direct_kernel(const DT* __restrict__ qhat, const DT* __restrict__ khat,
                                                     int64_t rows2, int H, int n, int k, uint64_t* __restrict__ cand,
                                                     int cs, int32_t* __restrict__ count) {
  __shared__ float qs[4][DH];
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r2 = (int64_t)blockIdx.x * 4 + wv;
  if (r2 >= rows2) return;
  exhaustive_row<DT, DH, LK>(qhat, khat, r2, H, n, k, cand, cs, count, qs[wv], lane);
}

// Every row exhaustively (few sub-keys for k, or query halves wider than the two MFMA passes
// are built for); lists of 32 keys per lane for k <= 32, else 64.
template <typename DT, int DH>
hipError_t launch_direct(const void* qhat, const void* khat, int64_t rows, int H, int n, int k, uint64_t* cand,
                         int32_t* count, hipStream_t s) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  const int cs = cand_slots(k);
  if (k <= 32)
    direct_kernel<DT, DH, 32><<<grid, 256, 0, s>>>((const DT*)qhat, (const DT*)khat, rows, H, n, k, cand, cs, count);
  else
    direct_kernel<DT, DH, MAX_K><<<grid, 256, 0, s>>>((const DT*)qhat, (const DT*)khat, rows, H, n, k, cand, cs, count);
  return hipGetLastError();
}

// The fp8 bound pass, where built: bf16 workloads with 256-wide halves (a 32-sub-key fp8
// chunk then splits evenly over 4 or 8 waves).
template <typename DT, int DH>
constexpr bool fp8_bound_built() {
  return sizeof(DT) == 2 && DH == 256;
}

template <typename DT, int DH, int NW, int FR>
hipError_t launch_passes_nw(const void* qhat, const void* khat, int64_t T, int H, int n, int k, float* gmax,
                            float* theta, uint64_t* cand, int32_t* count, int cus, const Fp8Bound& fb, hipStream_t s) {
  const int64_t tiles = (T + 32 * FR * NW - 1) / (32 * FR * NW);
  int gshift = 0;
  while (((n + (8 << gshift) - 1) >> (3 + gshift)) > MAX_GROUPS) ++gshift;
  const int ngroups = (n + (8 << gshift) - 1) >> (3 + gshift);
  // Sub-key splits for batches that leave CUs without a block: about one block per CU,
  // each split a whole number of pass 1's store batches of NB groups (so its first group
  // starts a 16-byte aligned batch)
  const int nch = (n + CHUNK - 1) / CHUNK;
  const int64_t blocks1 = tiles * 2 * H;
  int splits = 1, cps = nch;
  if (blocks1 < cus) {
    const int NB = NW == 8 ? 4 : 8;
    const int align = gshift <= 2 ? NB / (4 >> gshift) : (1 << (gshift - 2)) * NB;
    const int want = (int)(cus / blocks1);
    int c = (nch + want - 1) / want;
    c = (c + align - 1) / align * align;
    cps = c < nch ? c : nch;
    splits = (nch + cps - 1) / cps;
  }
  const dim3 grid((unsigned)(tiles * splits * 2 * H));
  const int64_t rows = T * H * 2;
  const int cs = cand_slots(k);
  hipError_t e;
  // too few groups for k and the bound prunes little: every row exhaustively.  k > 32 takes the
  // passes from k + 32 groups (at most 128 are formed), where the bound still leaves about
  // 100-190 candidates per row against 256 slots
  if (ngroups < (k <= 32 ? 2 * k : k + 32)) return launch_direct<DT, DH>(qhat, khat, rows, H, n, k, cand, count, s);
  const bool fp8 = fb.q8 != nullptr;
  if (fp8 && !fp8_bound_built<DT, DH>()) return hipErrorInvalidValue;
  // without split sub-key ranges pass 1 writes theta itself
  ThetaArgs ta;
  if (splits == 1) {
    ta.theta = theta;
    ta.k = k;
    ta.qn = fp8 ? fb.qn : nullptr;
    ta.kmax = fb.kmax;
    ta.eta = FP8_BOUND_ETA;
  }
#define PKM_P1(G)                                                                                                 \
  do {                                                                                                            \
    if constexpr (fp8_bound_built<DT, DH>()) {                                                                    \
      if (fp8) {                                                                                                  \
        pass1_kernel<uint8_t, DH, G, NW, FR><<<grid, 64 * NW, 0, s>>>((const uint8_t*)fb.q8, (const uint8_t*)fb.k8, T, \
                                                                      H, n, splits, cps, gmax,                    \
                                                                      splits > 1 ? count : nullptr, ta);          \
        break;                                                                                                    \
      }                                                                                                           \
    }                                                                                                             \
    pass1_kernel<DT, DH, G, NW, FR><<<grid, 64 * NW, 0, s>>>((const DT*)qhat, (const DT*)khat, T, H, n, splits, cps,   \
                                                             gmax, splits > 1 ? count : nullptr, ta);             \
  } while (0)
  switch (gshift) {
    case 0: PKM_P1(0); break;
    case 1: PKM_P1(1); break;
    case 2: PKM_P1(2); break;
    case 3: PKM_P1(3); break;
    case 4: PKM_P1(4); break;
    case 5: PKM_P1(5); break;
    case 6: PKM_P1(6); break;   // groups of 512: every n_sub with n_sub^2 < 2^31
    default: return hipErrorInvalidValue;  // n_sub > 128 * 512: rejected at create
  }
#undef PKM_P1
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (splits > 1) {
    theta_kernel<<<dim3((unsigned)((rows + 3) / 4)), 256, 0, s>>>(gmax, rows, ngroups, k, theta, fp8 ? fb.qn : nullptr,
                                                                   fb.kmax, 2 * H, FP8_BOUND_ETA);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (splits > 1) {
    // 8-wave blocks of 64-token waves are taken only when every CU gets one, so they never
    // split (and their LDS leaves no room for the stashes)
    if constexpr (NW == 8 && FR == 2) return hipErrorInvalidValue;
    else
      pass2_kernel<DT, DH, NW, FR, true><<<grid, 64 * NW, 0, s>>>((const DT*)qhat, (const DT*)khat, T, H, n, k, splits,
                                                                  cps, theta, cand, count, cs / 2);
  } else
    pass2_kernel<DT, DH, NW, FR, false><<<grid, 64 * NW, 0, s>>>((const DT*)qhat, (const DT*)khat, T, H, n, k, 1, nch,
                                                                 theta, cand, count, cs / 2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t scan_waves = (rows + 63) / 64;
  const int64_t ob = (scan_waves + 3) / 4 < 1024 ? (scan_waves + 3) / 4 : 1024;
  if (k <= 32)
    overflow_kernel<DT, DH, 32><<<dim3((unsigned)ob), 256, 0, s>>>((const DT*)qhat, (const DT*)khat, rows, H, n, k, cand,
                                                                   cs, count);
  else
    overflow_kernel<DT, DH, MAX_K><<<dim3((unsigned)ob), 256, 0, s>>>((const DT*)qhat, (const DT*)khat, rows, H, n, k,
                                                                      cand, cs, count);
  return hipGetLastError();
}

// 8-wave blocks where a chunk splits evenly over 8 waves: 64 tokens per wave if the batch
// gives every CU a block of them, else 32 (a block of 256 tokens; two waves per SIMD beat
// the 4-wave blocks of 64-token waves with the same block count, one wave per SIMD, by
// 25-30% at 1,024-8,192 tokens).  Else 4-wave blocks of 64-token waves.
template <typename DT, int DH>
constexpr bool eight_waves_built() {
  return (CHUNK * DH * (int)sizeof(DT) / 16) % (64 * 8) == 0;
}

template <typename DT, int DH>
hipError_t launch_passes(const void* qhat, const void* khat, int64_t T, int H, int n, int k, float* gmax, float* theta,
                         uint64_t* cand, int32_t* count, const Fp8Bound& fb, hipStream_t s) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      c = 256;
    cus = c;
  }
  if constexpr (eight_waves_built<DT, DH>()) {
    if ((T + 511) / 512 * 2 * H >= cus)
      return launch_passes_nw<DT, DH, 8, 2>(qhat, khat, T, H, n, k, gmax, theta, cand, count, cus, fb, s);
    return launch_passes_nw<DT, DH, 8, 1>(qhat, khat, T, H, n, k, gmax, theta, cand, count, cus, fb, s);
  } else {
    return launch_passes_nw<DT, DH, 4, 2>(qhat, khat, T, H, n, k, gmax, theta, cand, count, cus, fb, s);
  }
}

}  // namespace

hipError_t launch_score_candidates(const void* qhat, const void* khat, int64_t T, int H, int d_h, int n, int k,
                                   int dtype, float* gmax, float* theta, uint64_t* cand, int32_t* count,
                                   const Fp8Bound& fb, hipStream_t s) {
  if (T == 0) return hipSuccess;
#define PKM_PASSES(DT, DHV) return launch_passes<DT, DHV>(qhat, khat, T, H, n, k, gmax, theta, cand, count, fb, s)
  if (dtype == DT_BF16) {
    switch (d_h) {
      case 64: PKM_PASSES(uint16_t, 64);
      case 128: PKM_PASSES(uint16_t, 128);
      case 256: PKM_PASSES(uint16_t, 256);
    }
  } else {
    switch (d_h) {
      case 64: PKM_PASSES(float, 64);
      case 128: PKM_PASSES(float, 128);
      // fp32 halves wider than 128: the two MFMA passes would hold 256 query floats per lane,
      // so every row is scored exhaustively instead
      case 256: return launch_direct<float, 256>(qhat, khat, T * H * 2, H, n, k, cand, count, s);
    }
  }
#undef PKM_PASSES
  return hipErrorInvalidValue;
}

}  // namespace pkm
