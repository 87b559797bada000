// Dense GEMMs of the forward: the query projection q = x W_q, and the two Memory+
// products ("Memory Layers at Scale" digest, Memory+ block: out = (y * silu(x W1)) W2):
// z = x W1 in fp32 (the gate's elementwise part y * silu(z) is fused into the gather,
// which writes g) and out = g W2.
//
// C[M, N] = A[M, K] * Bt[N, K]^T: both operands are K-contiguous (the weights are
// transposed once at create), fp32 accumulation.
//  * bf16: matrix cores, v_mfma_f32_32x32x16_bf16.  Block tile 256 x 128 (128 x 128 for
//    small problems) with K-tiles of 32, four waves in a 2 x 2 arrangement, each wave
//    (BM/2) x (BN/2) (4 x 2 MFMA tiles at 256 x 128, so each 16-byte LDS operand read
//    feeds 1.33 MFMAs on average).  K-tiles reach padded LDS rows by direct global->LDS
//    loads into a double buffer; two blocks share a CU.
//  * fp32: a plain SIMT tile (64 x 64 x 16, 4 x 4 per thread) for the fp32 workloads.
#include "kernels.hpp"

namespace pkm {

namespace {

// Block tile BM x BN, four waves in a 2 x 2 grid, each wave (BM/2) x (BN/2) made of
// 32 x 32 MFMA tiles.  A and B K-tiles reach LDS by direct global->LDS loads
// (global_load_lds_dwordx4: each wave instruction fills 64 consecutive 16-byte LDS
// units) into a double buffer of padded rows (5 units of 16 bytes per 4 data units, so
// the MFMA operand reads are free of bank conflicts); a lane whose unit is padding
// loads a harmless in-bounds address.  One barrier per K-tile.
template <int BM, int BN, int EPI>
__global__ void __launch_bounds__(256, 2) gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ Bt, void* __restrict__ C,
                                                           int64_t M, int N, int K) {
  constexpr int WM = BM / 2, WN = BN / 2;      // wave tile
  constexpr int TM = WM / 32, TN = WN / 32;    // MFMA tiles per wave
  constexpr int BKT = 32;                      // K per LDS tile
  constexpr int RU = BKT / 8 + 1;              // 16-byte units per padded LDS row (4 data + 1 pad)
  constexpr int AUN = BM * RU, BUN = BN * RU;  // units per tile
  constexpr int AL = (AUN + 255) / 256, BL = (BUN + 255) / 256;  // loads per wave (4 waves x 64 lanes)
  __shared__ __attribute__((aligned(16))) uint8_t As[2][AL * 256 * 16];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BL * 256 * 16];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;

  // LDS unit p of a tile holds row p / RU, 16-byte column p % RU (column 4 = padding,
  // filled with a copy of column 3 and never read).  Rows past M / N read row 0 instead:
  // their products only reach outputs that are never stored.  K is a multiple of 32
  // (checked when the handle is created), so every column is real.
  auto fetch = [&](int k0, int buf) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int p = (wv * AL + i) * 64 + lane;
      int r = p / RU, cu = p - r * RU;
      int64_t gm = m0 + r;
      gm = (gm < M && p < AUN) ? gm : 0;
      cu = cu < 4 ? cu : 3;
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(A + gm * K + k0 + cu * 8),
          (void __attribute__((address_space(3)))*)(As[buf] + (wv * AL + i) * 64 * 16), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int p = (wv * BL + i) * 64 + lane;
      int r = p / RU, cu = p - r * RU;
      int gn = n0 + r;
      gn = (gn < N && p < BUN) ? gn : 0;
      cu = cu < 4 ? cu : 3;
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(Bt + (int64_t)gn * K + k0 + cu * 8),
          (void __attribute__((address_space(3)))*)(Bs[buf] + (wv * BL + i) * 64 * 16), 16, 0, 0);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  const int nk = K / BKT;
  fetch(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads have landed in LDS
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    // the other buffer was last read in the previous K-tile, before the barrier that ended it
    if (kt + 1 < nk) fetch((kt + 1) * BKT, buf ^ 1);
    const uint8_t* as = As[buf];
    const uint8_t* bs = Bs[buf];
#pragma unroll
    for (int kk = 0; kk < BKT / 16; ++kk) {
      bf16x8 af[TM], bfr[TN];
      const int cu = kk * 2 + (lane >> 5);  // 16-byte column of this lane's 8 k-values
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *(const bf16x8*)(as + ((wm * WM + i * 32 + (lane & 31)) * RU + cu) * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *(const bf16x8*)(bs + ((wn * WN + j * 32 + (lane & 31)) * RU + cu) * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }

  // epilogue: lane holds column n = .. + lane % 32 and 16 rows of each 32 x 32 tile
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * WN + j * 32 + (lane & 31);
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m >= M) continue;
        const float v = acc[i][j][r];
        const int64_t o = m * N + n;
        if (EPI == EPI_STORE_F32) {
          ((float*)C)[o] = v;
        } else {
          ((uint16_t*)C)[o] = f32_to_bf16(v);
        }
      }
    }
  }
}

__global__ void __launch_bounds__(256) gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ Bt,
                                                       float* __restrict__ C, int64_t M, int N, int K) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * 64;
  const int n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    // 64 rows x 16 k of each operand: 1024 elements, 4 per thread
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * 256;
      const int r = e >> 4, kc = e & 15;
      const int64_t gm = m0 + r;
      const int gn = n0 + r;
      As[kc][r] = (gm < M && k0 + kc < K) ? A[gm * K + k0 + kc] : 0.f;
      Bs[kc][r] = (gn < N && k0 + kc < K) ? Bt[(int64_t)gn * K + k0 + kc] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kc = 0; kc < 16; ++kc) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kc][ty * 4 + i];
        b[i] = Bs[kc][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      const int64_t o = m * N + n;
      C[o] = acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_gemm(const void* A, const void* Bt, void* C, int64_t M, int N, int K, int dtype, int epi,
                       hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (dtype == DT_BF16) {
    const uint16_t* a = (const uint16_t*)A;
    const uint16_t* b = (const uint16_t*)Bt;
    // large problems: 256 x 128 block tiles; small ones keep more blocks with 128 x 128
    const bool big = M >= 4096 && N >= 512;
#define PKM_GEMM(BMV, BNV, E)                                                                            \
  gemm_bf16_kernel<BMV, BNV, E><<<dim3((unsigned)((N + BNV - 1) / BNV), (unsigned)((M + BMV - 1) / BMV)), 256, 0, s>>>( \
      a, b, C, M, N, K)
    if (big) {
      if (epi == EPI_STORE_F32) PKM_GEMM(256, 128, EPI_STORE_F32);
      else PKM_GEMM(256, 128, EPI_STORE_DT);
    } else {
      if (epi == EPI_STORE_F32) PKM_GEMM(128, 128, EPI_STORE_F32);
      else PKM_GEMM(128, 128, EPI_STORE_DT);
    }
#undef PKM_GEMM
  } else {
    dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    const float* a = (const float*)A;
    const float* b = (const float*)Bt;
    gemm_f32_kernel<<<grid, 256, 0, s>>>(a, b, (float*)C, M, N, K);
  }
  return hipGetLastError();
}

}  // namespace pkm
