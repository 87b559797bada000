// Dense GEMMs of the forward: the query projection q = x W_q, and the two Memory+
// products ("Memory Layers at Scale" digest, Memory+ block: out = (y * silu(x W1)) W2):
// z = x W1 (the gate's elementwise part y * silu(z) is fused into the gather, which writes
// g) and out = g W2.  The bf16 products store their result in bf16 (the projection's q
// and z too: 15-20% faster than fp32 output at 16,384 x 4,096 x 2,048).
//
// C[M, N] = A[M, K] * Bt[N, K]^T: both operands are K-contiguous (the weights are
// transposed once at create), fp32 accumulation.
//  * bf16: these are plain GEMMs (no fused epilogue), so they go to hipBLASLt, which on
//    MI355X runs the 16384 x 2048 x 2048 shapes at 1.0-1.35 PFLOP/s against 0.8 for the
//    hand-written MFMA tiles this file held before.  The algorithm (the heuristic's first,
//    no workspace) is chosen once per device, (N, K, output type) and power-of-two bucket of
//    M, by a heuristic query for the bucket's largest M: the query is host work of about
//    0.1 s, so a batch size seen for the first time costs it only when its bucket is new, and
//    the number of queries stays bounded (at most 25 buckets per shape).  A plan for an exact
//    M (its layouts and the bucket's algorithm, checked to support that M, else the
//    heuristic's choice for it) is kept in a small cache, least recently used first out.
//    Host threads share the handle, the caches and the plans under one lock, which is also held
//    while a product is enqueued.
//    All candidate algorithms for these shapes were checked to be bitwise deterministic.
//  * fp32: a plain SIMT tile (64 x 64 x 16, 4 x 4 per thread) for the fp32 workloads.
#include <hipblaslt/hipblaslt-ext.hpp>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <memory>
#include <mutex>
#include <tuple>

#include "kernels.hpp"

namespace pkm {

namespace {

__global__ void __launch_bounds__(256) gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ Bt,
                                                       float* __restrict__ C, int64_t M, int N, int K) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  // token tiles on the grid's x dimension (2^31 - 1 blocks; y holds at most 65,536)
  const int64_t m0 = (int64_t)blockIdx.x * 64;
  const int n0 = blockIdx.y * 64;
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

// hipBLASLt is column-major: C[M, N] row-major is the column-major N x M matrix
// Bt^T(op T on the column-major K x N view of Bt) times A (the column-major K x M view of A).
struct LtPlan {
  LtPlan() = default;
  LtPlan(const LtPlan&) = delete;
  LtPlan& operator=(const LtPlan&) = delete;
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo;
  ~LtPlan() {
    if (lc) hipblasLtMatrixLayoutDestroy(lc);
    if (lb) hipblasLtMatrixLayoutDestroy(lb);
    if (la) hipblasLtMatrixLayoutDestroy(la);
    if (op) hipblasLtMatmulDescDestroy(op);
  }
};

// (device, M, N, K, out fp32); the algorithm cache's M is the bucket's largest M
typedef std::tuple<int, int64_t, int, int, int> PlanKey;
constexpr size_t MAX_PLANS = 64;

// The caches live until the process ends and are never destroyed (like the hipBLASLt
// handles): at exit, a destructor calling into hipBLASLt could run after its own teardown.
// Evicted plans are destroyed while the process runs, once no launch holds them.
std::mutex g_lt_mu;
auto& g_lt = *new std::map<int, hipblasLtHandle_t>;                       // per device
auto& g_algos = *new std::map<PlanKey, hipblasLtMatmulAlgo_t>;            // per bucket of M
auto& g_plans = *new std::map<PlanKey, std::pair<std::shared_ptr<const LtPlan>, uint64_t>>;  // exact M, last use
uint64_t g_tick = 0;

// descriptors of C[M, N] = A[M, K] Bt[N, K]^T with bf16 operands; false on failure
bool make_descs(LtPlan& P, int64_t M, int N, int K, bool out_f32) {
  bool ok = hipblasLtMatmulDescCreate(&P.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
  const hipblasOperation_t tA = HIPBLAS_OP_T, tB = HIPBLAS_OP_N;
  ok = ok && hipblasLtMatmulDescSetAttribute(P.op, HIPBLASLT_MATMUL_DESC_TRANSA, &tA, sizeof tA) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatmulDescSetAttribute(P.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tB, sizeof tB) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&P.la, HIP_R_16BF, K, N, K) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&P.lb, HIP_R_16BF, K, M, K) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&P.lc, out_f32 ? HIP_R_32F : HIP_R_16BF, N, M, N) == HIPBLAS_STATUS_SUCCESS;
  return ok;
}

// the heuristic's first algorithm (no workspace) for the plan's shape; false if none
bool heuristic_algo(hipblasLtHandle_t h, const LtPlan& P, hipblasLtMatmulAlgo_t* algo) {
  hipblasLtMatmulPreference_t pref = nullptr;
  bool ok = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
  const uint64_t no_ws = 0;
  ok = ok && hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &no_ws,
                                                   sizeof no_ws) == HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulHeuristicResult_t res[1];
  int got = 0;
  ok = ok && hipblasLtMatmulAlgoGetHeuristic(h, P.op, P.la, P.lb, P.lc, P.lc, pref, 1, res, &got) ==
                 HIPBLAS_STATUS_SUCCESS && got > 0;
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (ok) *algo = res[0].algo;
  return ok;
}

// the largest M of M's bucket: the next power of two (M >= 1)
int64_t bucket_top(int64_t M) {
  int64_t b = 1;
  while (b < M) b <<= 1;
  return b;
}

hipError_t lt_plan(int dev, int64_t M, int N, int K, bool out_f32, hipblasLtHandle_t* h,
                   std::shared_ptr<const LtPlan>* plan) {
  std::lock_guard<std::mutex> lock(g_lt_mu);
  auto hit = g_lt.find(dev);
  if (hit == g_lt.end()) {
    hipblasLtHandle_t lt = nullptr;
    if (hipblasLtCreate(&lt) != HIPBLAS_STATUS_SUCCESS) return hipErrorInitializationError;
    hit = g_lt.emplace(dev, lt).first;
  }
  *h = hit->second;
  const PlanKey key = std::make_tuple(dev, M, N, K, out_f32 ? 1 : 0);
  auto p = g_plans.find(key);
  if (p != g_plans.end()) {
    p->second.second = ++g_tick;
    *plan = p->second.first;
    return hipSuccess;
  }
  // the bucket's algorithm, from a heuristic query for the bucket's largest M
  const PlanKey bkey = std::make_tuple(dev, bucket_top(M), N, K, out_f32 ? 1 : 0);
  auto a = g_algos.find(bkey);
  if (a == g_algos.end()) {
    LtPlan B;
    hipblasLtMatmulAlgo_t algo;
    if (!make_descs(B, bucket_top(M), N, K, out_f32) || !heuristic_algo(*h, B, &algo)) return hipErrorNotSupported;
    a = g_algos.emplace(bkey, algo).first;
  }
  auto P = std::make_shared<LtPlan>();
  if (!make_descs(*P, M, N, K, out_f32)) return hipErrorNotSupported;
  P->algo = a->second;
  size_t ws = 0;
  const float alpha = 1.0f, beta = 0.0f;
  if (hipblaslt_ext::matmulIsAlgoSupported(*h, P->op, &alpha, P->la, P->lb, &beta, P->lc, P->lc, P->algo, ws) !=
          HIPBLAS_STATUS_SUCCESS || ws != 0) {
    // the bucket's choice does not take this M (or would need a workspace): the heuristic's for it
    if (!heuristic_algo(*h, *P, &P->algo)) return hipErrorNotSupported;
  }
  if (g_plans.size() >= MAX_PLANS) {  // evict the least recently used; launches holding it keep it alive
    auto old = g_plans.begin();
    for (auto it = g_plans.begin(); it != g_plans.end(); ++it)
      if (it->second.second < old->second.second) old = it;
    g_plans.erase(old);
  }
  g_plans.emplace(key, std::make_pair(std::shared_ptr<const LtPlan>(P), ++g_tick));
  *plan = P;
  return hipSuccess;
}

}  // namespace

hipError_t launch_gemm(const void* A, const void* Bt, void* C, int64_t M, int N, int K, int dtype, int epi,
                       hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (dtype == DT_BF16) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    hipblasLtHandle_t h;
    std::shared_ptr<const LtPlan> P;
    if ((e = lt_plan(dev, M, N, K, epi == EPI_STORE_F32, &h, &P)) != hipSuccess) return e;
    const float alpha = 1.0f, beta = 0.0f;
    hipblasStatus_t st;
    {  // host threads share one hipBLASLt handle per device: its calls (enqueue only) are serialised
      std::lock_guard<std::mutex> lock(g_lt_mu);
      st = hipblasLtMatmul(h, P->op, &alpha, Bt, P->la, A, P->lb, &beta, C, P->lc, C, P->lc, &P->algo, nullptr, 0, s);
    }
    return st == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
  } else {
    dim3 grid((unsigned)((M + 63) / 64), (unsigned)((N + 63) / 64));
    const float* a = (const float*)A;
    const float* b = (const float*)Bt;
    gemm_f32_kernel<<<grid, 256, 0, s>>>(a, b, (float*)C, M, N, K);
  }
  return hipGetLastError();
}

}  // namespace pkm
