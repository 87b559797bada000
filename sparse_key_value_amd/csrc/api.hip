// C ABI of the product-key memory forward: validation, workspace carving, and the
// launch sequence on the caller's stream.  Host code only; the kernels live in the
// other sources of this directory.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "layout.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define PKM_HIP(call)                                                                       \
  do {                                                                                      \
    hipError_t e_ = (call);                                                                 \
    if (e_ != hipSuccess) return fail(PKM_EHIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

int check_device() {
  int dev = 0;
  PKM_HIP(hipGetDevice(&dev));
  hipDeviceProp_t p;
  PKM_HIP(hipGetDeviceProperties(&p, dev));
  if (strncmp(p.gcnArchName, "gfx950", 6) != 0)
    return fail(PKM_EUNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev, p.gcnArchName);
  return PKM_OK;
}

}  // namespace

struct pkm_handle {
  pkm_config cfg;
  int d_h = 0;
  const void* values = nullptr;
  uint8_t* ws = nullptr;
  pkm::Layout L;
  // stage timing: max_rec records of PKM_NUM_STAGES boundary events each
  int max_rec = 0, next = 0, count = 0;
  std::vector<hipEvent_t> ev;

  template <typename T = void>
  T* at(size_t off) const { return (T*)(ws + off); }
};

namespace {

void destroy_events(pkm_handle* h) {
  for (hipEvent_t e : h->ev)
    if (e) (void)hipEventDestroy(e);
  h->ev.clear();
  h->max_rec = h->next = h->count = 0;
}

struct Timer {
  pkm_handle* h;
  hipStream_t s;
  int slot;
  explicit Timer(pkm_handle* h_, hipStream_t s_) : h(h_), s(s_), slot(h_->max_rec ? h_->next : -1) {}
  hipError_t mark(int boundary) {
    if (slot < 0) return hipSuccess;
    return hipEventRecord(h->ev[(size_t)slot * PKM_NUM_STAGES + boundary], s);
  }
  void commit() {
    if (slot < 0) return;
    h->next = (h->next + 1) % h->max_rec;
    if (h->count < h->max_rec) ++h->count;
  }
};

#define PKM_LAUNCH(call)                                                                              \
  do {                                                                                                \
    hipError_t e_ = (call);                                                                           \
    if (e_ != hipSuccess) return fail(PKM_EHIP, "launch %s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)

int run_select(pkm_handle* h, const void* qhat, int64_t T, int32_t* hidx, float* hsc, int32_t* idx, float* sc,
               float* w, hipStream_t s, Timer* tm) {
  const pkm_config& c = h->cfg;
  PKM_LAUNCH(pkm::launch_score_topk(qhat, h->at(h->L.khat), T, c.n_heads, h->d_h, c.n_sub, c.k, c.dtype, hidx, hsc, s));
  if (tm) PKM_LAUNCH(tm->mark(3));
  PKM_LAUNCH(pkm::launch_combine(hidx, hsc, T, c.n_heads, c.n_sub, c.k, idx, sc, w, s));
  if (tm) PKM_LAUNCH(tm->mark(4));
  return PKM_OK;
}

int run_forward(pkm_handle* h, const void* x, int64_t T, void* out, const pkm_debug_ptrs* dbg, int32_t* idx_out,
                float* w_out, hipStream_t s) {
  if (!h) return fail(PKM_EINVAL, "handle is NULL");
  const pkm_config& c = h->cfg;
  if (T < 0 || T > c.max_tokens) return fail(PKM_EINVAL, "T = %lld outside [0, max_tokens = %lld]", (long long)T, (long long)c.max_tokens);
  if (T == 0) return PKM_OK;
  if (!x || !out) return fail(PKM_EINVAL, "x and out must not be NULL");
  const pkm::Layout& L = h->L;
  const int H = c.n_heads, dq = c.d_query, k = c.k;
  const size_t eb = c.dtype == PKM_BF16 ? 2 : 4;

  Timer tm(h, s);
  PKM_LAUNCH(tm.mark(0));
  // a1: q = x W_q (fp32)
  PKM_LAUNCH(pkm::launch_gemm(x, h->at(L.wqT), h->at(L.q), nullptr, T, H * dq, c.d_model, c.dtype, pkm::EPI_STORE_F32, s));
  PKM_LAUNCH(tm.mark(1));
  // a2: qk-norm over each head's d_q, stored in dtype; the halves are the two contiguous halves
  PKM_LAUNCH(pkm::launch_rownorm(h->at(L.q), 1, h->at(L.qhat), c.dtype, T * H, dq, c.qk_norm, c.norm_eps, s));
  PKM_LAUNCH(tm.mark(2));
  // a3-a6: scoring + per-half top-k, combine + final top-k + softmax
  int32_t* idx = h->at<int32_t>(L.idx);
  float* w = h->at<float>(L.w);
  int rc = run_select(h, h->at(L.qhat), T, h->at<int32_t>(L.hidx), h->at<float>(L.hsc), idx, h->at<float>(L.sc), w, s, &tm);
  if (rc) return rc;
  // a7: weighted EmbeddingBag of the H*k rows of every token
  const int64_t N = (int64_t)c.n_sub * c.n_sub;
  float* ydbg = dbg ? dbg->y : nullptr;
  if (c.memory_plus) {
    float* y = ydbg ? ydbg : h->at<float>(L.y);
    PKM_LAUNCH(pkm::launch_gather(h->values, N, c.d_value, c.dtype, idx, w, T, H * k, y, 0, s));
    PKM_LAUNCH(tm.mark(5));
    // a8: g = y * silu(x W1) in dtype, out = g W2
    PKM_LAUNCH(pkm::launch_gemm(x, h->at(L.w1T), h->at(L.g), y, T, c.d_value, c.d_model, c.dtype, pkm::EPI_GATE, s));
    PKM_LAUNCH(tm.mark(6));
    PKM_LAUNCH(pkm::launch_gemm(h->at(L.g), h->at(L.w2T), out, nullptr, T, c.d_model, c.d_value, c.dtype,
                                c.dtype == PKM_BF16 ? pkm::EPI_STORE_DT : pkm::EPI_STORE_F32, s));
    PKM_LAUNCH(tm.mark(7));
  } else {
    if (ydbg) {
      PKM_LAUNCH(pkm::launch_gather(h->values, N, c.d_value, c.dtype, idx, w, T, H * k, ydbg, 0, s));
      PKM_LAUNCH(pkm::launch_convert_f32(ydbg, out, T * c.d_value, c.dtype, s));
    } else {
      PKM_LAUNCH(pkm::launch_gather(h->values, N, c.d_value, c.dtype, idx, w, T, H * k, out, 1, s));
    }
    PKM_LAUNCH(tm.mark(5));
    PKM_LAUNCH(tm.mark(6));
    PKM_LAUNCH(tm.mark(7));
  }
  tm.commit();

  const size_t nsel = (size_t)T * H * k;
  if (idx_out) PKM_HIP(hipMemcpyAsync(idx_out, idx, nsel * 4, hipMemcpyDeviceToDevice, s));
  if (w_out) PKM_HIP(hipMemcpyAsync(w_out, w, nsel * 4, hipMemcpyDeviceToDevice, s));
  if (dbg) {
    if (dbg->qhat) PKM_HIP(hipMemcpyAsync(dbg->qhat, h->at(L.qhat), (size_t)T * H * dq * eb, hipMemcpyDeviceToDevice, s));
    if (dbg->half_idx) PKM_HIP(hipMemcpyAsync(dbg->half_idx, h->at(L.hidx), 2 * nsel * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->half_score) PKM_HIP(hipMemcpyAsync(dbg->half_score, h->at(L.hsc), 2 * nsel * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->idx) PKM_HIP(hipMemcpyAsync(dbg->idx, idx, nsel * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->score) PKM_HIP(hipMemcpyAsync(dbg->score, h->at(L.sc), nsel * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->w) PKM_HIP(hipMemcpyAsync(dbg->w, w, nsel * 4, hipMemcpyDeviceToDevice, s));
  }
  return PKM_OK;
}

}  // namespace

extern "C" {

const char* pkm_last_error(void) { return g_err.c_str(); }

size_t pkm_workspace_size(const pkm_config* cfg) {
  std::string why = pkm::check_config(cfg);
  if (!why.empty()) {
    fail(PKM_EINVAL, "invalid config: %s", why.c_str());
    return 0;
  }
  return pkm::make_layout(cfg).total;
}

int pkm_create(const pkm_config* cfg, const void* W_q, const void* subkeys, const void* values, const void* W1,
               const void* W2, void* workspace, size_t ws_bytes, void* stream, pkm_handle** out) {
  if (!out) return fail(PKM_EINVAL, "out (handle pointer) is NULL");
  *out = nullptr;
  std::string why = pkm::check_config(cfg);
  if (!why.empty()) return fail(PKM_EINVAL, "invalid config: %s", why.c_str());
  if (!W_q || !subkeys || !values || !workspace) return fail(PKM_EINVAL, "W_q, subkeys, values and workspace must not be NULL");
  if (cfg->memory_plus && (!W1 || !W2)) return fail(PKM_EINVAL, "memory_plus needs W1 and W2");
  if (((uintptr_t)values & 15) != 0) return fail(PKM_EINVAL, "values must be 16-byte aligned");
  if (((uintptr_t)workspace & 255) != 0) return fail(PKM_EINVAL, "workspace must be 256-byte aligned");
  pkm::Layout L = pkm::make_layout(cfg);
  if (ws_bytes < L.total)
    return fail(PKM_EWORKSPACE, "workspace has %zu bytes, the config needs %zu", ws_bytes, L.total);
  int rc = check_device();
  if (rc) return rc;

  pkm_handle* h = new (std::nothrow) pkm_handle();
  if (!h) return fail(PKM_EINVAL, "out of host memory");
  h->cfg = *cfg;
  h->d_h = cfg->d_query / 2;
  h->values = values;
  h->ws = (uint8_t*)workspace;
  h->L = L;
  hipStream_t s = (hipStream_t)stream;
  const pkm_config& c = *cfg;
  auto bail = [&](int code) {
    delete h;
    return code;
  };
  hipError_t e;
  // W_q [d_model, H*d_q] -> [H*d_q, d_model]
  if ((e = pkm::launch_transpose(W_q, h->at(L.wqT), c.d_model, c.n_heads * c.d_query, c.dtype, s)) != hipSuccess)
    return bail(fail(PKM_EHIP, "repack of W_q failed: %s", hipGetErrorString(e)));
  // fold qk-norm into the sub-keys: one row per (head, half, sub-key)
  if ((e = pkm::launch_rownorm(subkeys, c.dtype == PKM_F32, h->at(L.khat), c.dtype, (int64_t)c.n_heads * 2 * c.n_sub,
                               h->d_h, c.qk_norm, c.norm_eps, s)) != hipSuccess)
    return bail(fail(PKM_EHIP, "sub-key normalisation failed: %s", hipGetErrorString(e)));
  if (c.memory_plus) {
    if ((e = pkm::launch_transpose(W1, h->at(L.w1T), c.d_model, c.d_value, c.dtype, s)) != hipSuccess ||
        (e = pkm::launch_transpose(W2, h->at(L.w2T), c.d_value, c.d_model, c.dtype, s)) != hipSuccess)
      return bail(fail(PKM_EHIP, "repack of W1/W2 failed: %s", hipGetErrorString(e)));
  }
  *out = h;
  return PKM_OK;
}

int pkm_forward(pkm_handle* h, const void* x, int64_t T, void* out, int32_t* idx_out, float* w_out, void* stream) {
  return run_forward(h, x, T, out, nullptr, idx_out, w_out, (hipStream_t)stream);
}

int pkm_forward_debug(pkm_handle* h, const void* x, int64_t T, void* out, const pkm_debug_ptrs* dbg, void* stream) {
  return run_forward(h, x, T, out, dbg, nullptr, nullptr, (hipStream_t)stream);
}

int pkm_select(pkm_handle* h, const void* qhat, int64_t T, int32_t* half_idx, float* half_score, int32_t* idx,
               float* score, float* w, void* stream) {
  if (!h) return fail(PKM_EINVAL, "handle is NULL");
  if (T < 0 || T > h->cfg.max_tokens) return fail(PKM_EINVAL, "T = %lld outside [0, max_tokens]", (long long)T);
  if (T == 0) return PKM_OK;
  if (!qhat) return fail(PKM_EINVAL, "qhat must not be NULL");
  const pkm::Layout& L = h->L;
  return run_select(h, qhat, T, half_idx ? half_idx : h->at<int32_t>(L.hidx), half_score ? half_score : h->at<float>(L.hsc),
                    idx ? idx : h->at<int32_t>(L.idx), score ? score : h->at<float>(L.sc), w ? w : h->at<float>(L.w),
                    (hipStream_t)stream, nullptr);
}

int pkm_copy_normalized_subkeys(pkm_handle* h, void* dst, void* stream) {
  if (!h || !dst) return fail(PKM_EINVAL, "handle and dst must not be NULL");
  const size_t eb = h->cfg.dtype == PKM_BF16 ? 2 : 4;
  const size_t bytes = (size_t)h->cfg.n_heads * 2 * h->cfg.n_sub * h->d_h * eb;
  PKM_HIP(hipMemcpyAsync(dst, h->at(h->L.khat), bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream));
  return PKM_OK;
}

int pkm_embedding_bag(const void* table, int64_t n_rows, int32_t dim, int32_t dtype, const int32_t* idx, const float* w,
                      int64_t n_bags, int32_t bag_size, float* y, void* stream) {
  if (dtype != PKM_F32 && dtype != PKM_BF16) return fail(PKM_EINVAL, "dtype must be PKM_F32 or PKM_BF16");
  const int eb = dtype == PKM_BF16 ? 2 : 4;
  if (dim <= 0 || ((int64_t)dim * eb) % 16 != 0) return fail(PKM_EINVAL, "dim * sizeof(dtype) must be a positive multiple of 16");
  if (n_rows < 1) return fail(PKM_EINVAL, "n_rows must be >= 1");
  if (n_bags < 0 || n_bags > ((int64_t)1 << 31) - 1) return fail(PKM_EINVAL, "n_bags must be in [0, 2^31)");
  if (bag_size < 1) return fail(PKM_EINVAL, "bag_size must be >= 1");
  if (n_bags == 0) return PKM_OK;
  if (!table || !idx || !w || !y) return fail(PKM_EINVAL, "table, idx, w and y must not be NULL");
  if (((uintptr_t)table & 15) != 0) return fail(PKM_EINVAL, "table must be 16-byte aligned");
  PKM_LAUNCH(pkm::launch_gather(table, n_rows, dim, dtype, idx, w, n_bags, bag_size, y, 0, (hipStream_t)stream));
  return PKM_OK;
}

int pkm_enable_stage_timing(pkm_handle* h, int32_t max_records) {
  if (!h) return fail(PKM_EINVAL, "handle is NULL");
  if (max_records < 0 || max_records > 4096) return fail(PKM_EINVAL, "max_records must be in [0, 4096]");
  destroy_events(h);
  if (max_records == 0) return PKM_OK;
  h->ev.assign((size_t)max_records * PKM_NUM_STAGES, nullptr);
  for (hipEvent_t& e : h->ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      destroy_events(h);
      return fail(PKM_EHIP, "hipEventCreate: %s", hipGetErrorString(r));
    }
  }
  h->max_rec = max_records;
  return PKM_OK;
}

int pkm_stage_times(pkm_handle* h, int32_t stage, float* ms, int32_t n) {
  if (!h || !ms) return fail(PKM_EINVAL, "handle and ms must not be NULL");
  if (stage < 0 || stage >= PKM_NUM_STAGES) return fail(PKM_EINVAL, "stage must be in [0, %d)", PKM_NUM_STAGES);
  if (h->max_rec == 0) return fail(PKM_EINVAL, "stage timing is off (pkm_enable_stage_timing)");
  const int have = h->count < n ? h->count : n;
  const int first = (h->next - h->count + h->max_rec) % h->max_rec;  // oldest record
  const int skip = h->count - have;
  for (int i = 0; i < have; ++i) {
    const int slot = (first + skip + i) % h->max_rec;
    hipEvent_t* e = &h->ev[(size_t)slot * PKM_NUM_STAGES];
    const int b0 = stage == PKM_STAGE_TOTAL ? 0 : stage;
    const int b1 = stage == PKM_STAGE_TOTAL ? PKM_NUM_STAGES - 1 : stage + 1;
    PKM_HIP(hipEventSynchronize(e[b1]));
    PKM_HIP(hipEventElapsedTime(&ms[i], e[b0], e[b1]));
  }
  return have;
}

int pkm_destroy(pkm_handle* h) {
  if (!h) return fail(PKM_EINVAL, "handle is NULL");
  destroy_events(h);
  delete h;
  return PKM_OK;
}

}  // extern "C"
