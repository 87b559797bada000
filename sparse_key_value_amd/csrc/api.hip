// C ABI of the product-key memory forward: validation, workspace carving, and the
// launch sequence on the caller's stream.  Host code only; the kernels live in the
// other sources of this directory.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <string>
#include <vector>

#include "abi.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace pkm_abi {

namespace {
thread_local std::string g_err;
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int check_device() {
  int dev = 0;
  PKM_HIP(hipGetDevice(&dev));
  hipDeviceProp_t p;
  PKM_HIP(hipGetDeviceProperties(&p, dev));
  if (strncmp(p.gcnArchName, "gfx950", 6) != 0)
    return fail(PKM_EUNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev, p.gcnArchName);
  return PKM_OK;
}

const char* last_error() { return g_err.c_str(); }

int device_view(const void* p, const char* what, const void** out) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PKM_EINVAL, "%s: neither device memory nor pinned host memory", what);
  }
  if (at.type == hipMemoryTypeDevice) {
    *out = p;
    return PKM_OK;
  }
  if (at.type == hipMemoryTypeHost) {
    void* d = nullptr;
    PKM_HIP(hipHostGetDevicePointer(&d, const_cast<void*>(p), 0));
    if (!d) return fail(PKM_EINVAL, "%s: pinned host memory without a device mapping", what);
    *out = d;
    return PKM_OK;
  }
  return fail(PKM_EINVAL, "%s must be device memory or pinned host memory (e.g. hipHostMalloc)", what);
}

int require_device(const void* p, const char* what) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PKM_EINVAL, "%s is not device memory", what);
  }
  if (at.type != hipMemoryTypeDevice) return fail(PKM_EINVAL, "%s must be device memory", what);
  return PKM_OK;
}

}  // namespace pkm_abi

using pkm_abi::check_device;
using pkm_abi::fail;

struct pkm_handle {
  pkm_config cfg;
  int d_h = 0;   // d_query / 2
  int d_hp = 0;  // d_h padded for scoring: the stored width of query halves and sub-key rows
  bool fp8 = false;  // the bound pass scores in fp8 (pkm_set_score_bound)
  const void* values = nullptr;
  uint8_t* ws = nullptr;
  pkm::Layout L;
  // stage timing: max_rec records, each with (begin, end) events per stage
  int max_rec = 0, next = 0, count = 0;
  uint32_t stage_mask = (1u << PKM_NUM_STAGES) - 1u;  // bit s: stage s is recorded
  std::vector<uint32_t> rec_mask;  // the mask each record was taken with
  std::vector<hipEvent_t> ev;

  template <typename T = void>
  T* at(size_t off) const { return (T*)(ws + off); }
};

namespace {

constexpr int EV_PER_REC = PKM_NUM_STAGES * 2;

void destroy_timing(pkm_handle* h) {
  for (hipEvent_t e : h->ev)
    if (e) (void)hipEventDestroy(e);
  h->ev.clear();
  h->rec_mask.clear();
  h->max_rec = h->next = h->count = 0;
}

// HIP events around the stages of one forward, if timing is on and the stage is in the mask.
struct Timer {
  pkm_handle* h;
  int slot;
  explicit Timer(pkm_handle* h_) : h(h_), slot(h_->max_rec ? h_->next : -1) {
    if (slot >= 0) h->rec_mask[slot] = h->stage_mask;
  }
  hipError_t stage(int st, int end, hipStream_t s) {
    if (slot < 0 || !((h->rec_mask[slot] >> st) & 1u)) return hipSuccess;
    return hipEventRecord(h->ev[(size_t)slot * EV_PER_REC + st * 2 + end], s);
  }
  void commit() {
    if (slot < 0) return;
    h->next = (h->next + 1) % h->max_rec;
    if (h->count < h->max_rec) ++h->count;
  }
};

int run_select(pkm_handle* h, const void* qhat, int64_t T, int32_t* hidx, float* hsc, int32_t* idx, float* sc,
               float* w, hipStream_t s, Timer* tm) {
  const pkm_config& c = h->cfg;
  const pkm::Layout& L = h->L;
  if (tm) PKM_LAUNCH(tm->stage(PKM_STAGE_SCORE, 0, s));
  pkm::Fp8Bound fb;
  if (h->fp8) {
    fb.q8 = h->at(L.q8);
    fb.k8 = h->at(L.khat8);
    fb.qn = h->at<float>(L.qn);
    fb.kmax = h->at<float>(L.kmax);
  }
  PKM_LAUNCH(pkm::launch_score_candidates(qhat, h->at(L.khat), T, c.n_heads, h->d_hp, c.n_sub, c.k, c.dtype,
                                          h->at<float>(L.gmax), h->at<float>(L.theta), h->at<uint64_t>(L.cand),
                                          h->at<int32_t>(L.count), fb, s));
  if (tm) PKM_LAUNCH(tm->stage(PKM_STAGE_SCORE, 1, s));
  if (tm) PKM_LAUNCH(tm->stage(PKM_STAGE_COMBINE, 0, s));
  PKM_LAUNCH(pkm::launch_combine(h->at<uint64_t>(L.cand), h->at<int32_t>(L.count), T, c.n_heads, c.n_sub, c.k, hidx,
                                 hsc, idx, sc, w, s));
  if (tm) PKM_LAUNCH(tm->stage(PKM_STAGE_COMBINE, 1, s));
  return PKM_OK;
}

// The forward in order on `s`.  The per-half lists are written only when `halves` (a debug
// forward that asks for them): the forward itself needs only the final lists.  A debug y
// (fp32) comes from one more plain gather, whose arithmetic is the fused one's.
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
  const int64_t N = (int64_t)c.n_sub * c.n_sub;
  float* ydbg = dbg ? dbg->y : nullptr;
  const bool halves = dbg && (dbg->half_idx || dbg->half_score);
  void* q = h->at(L.q);  // [T, qz_cols] in the stored type
  int32_t* idx = h->at<int32_t>(L.idx);
  float* w = h->at<float>(L.w);

  Timer tm(h);
  PKM_LAUNCH(tm.stage(PKM_STAGE_TOTAL, 0, s));
  // a1: q = x W_q, stored in the model's type (bf16 or fp32) as a product in that type
  // returns it; with the Memory+ gate the same GEMM also computes z = x W1 (the first
  // product of a8) into the next d_v columns: one 16,384 x 4,096 product runs faster than
  // two of 16,384 x 2,048 on MI355X, and its bf16 output 15-20% faster than an fp32 one
  PKM_LAUNCH(tm.stage(PKM_STAGE_PROJECT, 0, s));
  PKM_LAUNCH(pkm::launch_gemm(x, h->at(L.wqT), q, T, (int)L.qz_cols, c.d_model, c.dtype, pkm::EPI_STORE_DT, s));
  PKM_LAUNCH(tm.stage(PKM_STAGE_PROJECT, 1, s));
  // a2: qk-norm over each head's d_q, stored in dtype; the halves are the two contiguous halves,
  // each stored in d_hp elements (zeros after d_h); for the fp8 bound also their e4m3 copies
  // and norms
  PKM_LAUNCH(tm.stage(PKM_STAGE_QNORM, 0, s));
  PKM_LAUNCH(pkm::launch_rownorm(q, c.dtype == PKM_F32, h->at(L.qhat), c.dtype, T * H, dq, c.qk_norm, c.norm_eps, s, H, L.qz_cols,
                                 h->d_h, h->d_hp, h->fp8 ? h->at<uint8_t>(L.q8) : nullptr,
                                 h->fp8 ? h->at<float>(L.qn) : nullptr));
  PKM_LAUNCH(tm.stage(PKM_STAGE_QNORM, 1, s));
  // a3-a6: scoring + per-half top-k, combine + final top-k + softmax
  int rc = run_select(h, h->at(L.qhat), T, halves ? h->at<int32_t>(L.hidx) : nullptr,
                      halves ? h->at<float>(L.hsc) : nullptr, idx, h->at<float>(L.sc), w, s, &tm);
  if (rc) return rc;
  // a7 (+ a8's elementwise part): with the gate, g = y * silu(z) in dtype; else y into out
  PKM_LAUNCH(tm.stage(PKM_STAGE_GATHER, 0, s));
  if (c.memory_plus) {
    const void* z = (const uint8_t*)q + (size_t)H * dq * eb;  // the columns of x W1
    PKM_LAUNCH(pkm::launch_gather(h->values, N, c.d_value, c.dtype, idx, w, T, H * k, h->at(L.g), 1, s, z, L.qz_cols,
                                  c.dtype == PKM_BF16));
    if (ydbg) PKM_LAUNCH(pkm::launch_gather(h->values, N, c.d_value, c.dtype, idx, w, T, H * k, ydbg, 0, s));
  } else if (ydbg) {
    PKM_LAUNCH(pkm::launch_gather(h->values, N, c.d_value, c.dtype, idx, w, T, H * k, ydbg, 0, s));
    PKM_LAUNCH(pkm::launch_convert_f32(ydbg, out, T * c.d_value, c.dtype, s));
  } else {
    PKM_LAUNCH(pkm::launch_gather(h->values, N, c.d_value, c.dtype, idx, w, T, H * k, out, 1, s));
  }
  PKM_LAUNCH(tm.stage(PKM_STAGE_GATHER, 1, s));
  // a8: out = g W2
  if (c.memory_plus) {
    PKM_LAUNCH(tm.stage(PKM_STAGE_GATE, 0, s));
    PKM_LAUNCH(pkm::launch_gemm(h->at(L.g), h->at(L.w2T), out, T, c.d_model, c.d_value, c.dtype,
                                c.dtype == PKM_BF16 ? pkm::EPI_STORE_DT : pkm::EPI_STORE_F32, s));
    PKM_LAUNCH(tm.stage(PKM_STAGE_GATE, 1, s));
  }
  PKM_LAUNCH(tm.stage(PKM_STAGE_TOTAL, 1, s));
  tm.commit();

  const size_t nsel = (size_t)T * H * k;
  if (idx_out) PKM_HIP(hipMemcpyAsync(idx_out, idx, nsel * 4, hipMemcpyDeviceToDevice, s));
  if (w_out) PKM_HIP(hipMemcpyAsync(w_out, w, nsel * 4, hipMemcpyDeviceToDevice, s));
  if (dbg) {
    if (dbg->qhat)  // [T, H, 2, d_h] from the padded rows
      PKM_HIP(hipMemcpy2DAsync(dbg->qhat, h->d_h * eb, h->at(L.qhat), h->d_hp * eb, h->d_h * eb, (size_t)T * H * 2,
                               hipMemcpyDeviceToDevice, s));
    if (dbg->half_idx) PKM_HIP(hipMemcpyAsync(dbg->half_idx, h->at(L.hidx), 2 * nsel * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->half_score) PKM_HIP(hipMemcpyAsync(dbg->half_score, h->at(L.hsc), 2 * nsel * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->idx) PKM_HIP(hipMemcpyAsync(dbg->idx, idx, nsel * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->score) PKM_HIP(hipMemcpyAsync(dbg->score, h->at(L.sc), nsel * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->w) PKM_HIP(hipMemcpyAsync(dbg->w, w, nsel * 4, hipMemcpyDeviceToDevice, s));
    const size_t rows = (size_t)T * H * 2;
    if (dbg->theta) PKM_HIP(hipMemcpyAsync(dbg->theta, h->at(L.theta), rows * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->counts) PKM_HIP(hipMemcpyAsync(dbg->counts, h->at(L.count), rows * 2 * 4, hipMemcpyDeviceToDevice, s));
  }
  return PKM_OK;
}

}  // namespace

extern "C" {

const char* pkm_last_error(void) { return pkm_abi::last_error(); }

size_t pkm_workspace_size(const pkm_config* cfg) {
  std::string why = pkm::check_config(cfg);
  if (!why.empty()) {
    fail(PKM_EINVAL, "invalid config: %s", why.c_str());
    return 0;
  }
  why = pkm::unsupported_reason(cfg);
  if (!why.empty()) {
    fail(PKM_EUNSUPPORTED, "unsupported config: %s", why.c_str());
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
  why = pkm::unsupported_reason(cfg);
  if (!why.empty()) return fail(PKM_EUNSUPPORTED, "unsupported config: %s", why.c_str());
  if (!W_q || !subkeys || !values || !workspace) return fail(PKM_EINVAL, "W_q, subkeys, values and workspace must not be NULL");
  if (cfg->memory_plus && (!W1 || !W2)) return fail(PKM_EINVAL, "memory_plus needs W1 and W2");
  if (((uintptr_t)values & 15) != 0) return fail(PKM_EINVAL, "values must be 16-byte aligned");
  if (((uintptr_t)workspace & 255) != 0) return fail(PKM_EINVAL, "workspace must be 256-byte aligned");
  pkm::Layout L = pkm::make_layout(cfg);
  if (ws_bytes < L.total)
    return fail(PKM_EWORKSPACE, "workspace has %zu bytes, the config needs %zu", ws_bytes, L.total);
  int rc = check_device();
  if (rc) return rc;
  if ((rc = pkm_abi::require_device(workspace, "workspace")) != PKM_OK) return rc;
  if ((rc = pkm_abi::require_device(W_q, "W_q")) != PKM_OK) return rc;
  if ((rc = pkm_abi::require_device(subkeys, "subkeys")) != PKM_OK) return rc;
  if (cfg->memory_plus) {
    if ((rc = pkm_abi::require_device(W1, "W1")) != PKM_OK) return rc;
    if ((rc = pkm_abi::require_device(W2, "W2")) != PKM_OK) return rc;
  }

  pkm_handle* h = new (std::nothrow) pkm_handle();
  if (!h) return fail(PKM_EINVAL, "out of host memory");
  h->cfg = *cfg;
  h->d_h = cfg->d_query / 2;
  h->d_hp = pkm::padded_half(h->d_h);
  h->fp8 = pkm::fp8_bound(cfg);
  const void* vview = nullptr;
  if ((rc = pkm_abi::device_view(values, "values", &vview)) != PKM_OK) {
    delete h;
    return rc;
  }
  h->values = vview;
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
  // fold qk-norm into the sub-keys: one row per (head, half, sub-key), stored in d_hp elements
  if ((e = pkm::launch_rownorm(subkeys, c.dtype == PKM_F32, h->at(L.khat), c.dtype, (int64_t)c.n_heads * 2 * c.n_sub,
                               h->d_h, c.qk_norm, c.norm_eps, s, 1, 0, h->d_h, h->d_hp)) != hipSuccess)
    return bail(fail(PKM_EHIP, "sub-key normalisation failed: %s", hipGetErrorString(e)));
  // the fp8 copy of the normalised sub-keys, their norms and the largest norm per (head, half)
  if (pkm::fp8_bound(cfg) &&
      (e = pkm::launch_fp8_rows(h->at(L.khat), h->at<uint8_t>(L.khat8), h->at<float>(L.knorm),
                                (int64_t)c.n_heads * 2 * c.n_sub, h->d_hp, h->at<float>(L.kmax), c.n_sub, s)) != hipSuccess)
    return bail(fail(PKM_EHIP, "fp8 sub-keys failed: %s", hipGetErrorString(e)));
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
  hipStream_t s = (hipStream_t)stream;
  if (h->d_hp != h->d_h) {  // the caller's [T, H, 2, d_h] rows, padded to the scoring width
    PKM_LAUNCH(pkm::launch_pad_rows(qhat, h->at(L.qhat), T * h->cfg.n_heads * 2, h->d_h, h->d_hp, h->cfg.dtype, s));
    qhat = h->at(L.qhat);
  }
  if (h->fp8)  // the e4m3 copy and the norms of the query halves, for the bound pass
    PKM_LAUNCH(pkm::launch_fp8_rows(qhat, h->at<uint8_t>(L.q8), h->at<float>(L.qn), T * h->cfg.n_heads * 2, h->d_hp,
                                    nullptr, 1, s));
  return run_select(h, qhat, T, half_idx ? half_idx : h->at<int32_t>(L.hidx), half_score ? half_score : h->at<float>(L.hsc),
                    idx ? idx : h->at<int32_t>(L.idx), score ? score : h->at<float>(L.sc), w ? w : h->at<float>(L.w),
                    s, nullptr);
}

int pkm_copy_normalized_subkeys(pkm_handle* h, void* dst, void* stream) {
  if (!h || !dst) return fail(PKM_EINVAL, "handle and dst must not be NULL");
  const size_t eb = h->cfg.dtype == PKM_BF16 ? 2 : 4;
  // [H, 2, n_sub, d_h] from the padded rows
  PKM_HIP(hipMemcpy2DAsync(dst, h->d_h * eb, h->at(h->L.khat), h->d_hp * eb, h->d_h * eb,
                           (size_t)h->cfg.n_heads * 2 * h->cfg.n_sub, hipMemcpyDeviceToDevice, (hipStream_t)stream));
  return PKM_OK;
}

int pkm_embedding_bag(const void* table, int64_t n_rows, int32_t dim, int32_t dtype, const int32_t* idx, const float* w,
                      int64_t n_bags, int32_t bag_size, float* y, void* stream) {
  if (dtype != PKM_F32 && dtype != PKM_BF16) return fail(PKM_EINVAL, "dtype must be PKM_F32 or PKM_BF16");
  const int eb = dtype == PKM_BF16 ? 2 : 4;
  if (dim <= 0 || ((int64_t)dim * eb) % 16 != 0) return fail(PKM_EINVAL, "dim * sizeof(dtype) must be a positive multiple of 16");
  // a row's 16-byte slices go to blocks of 256 lanes along the launch grid's y dimension (at most
  // 65,536 blocks): 2^24 elements need at most 16,384
  if (dim > (1 << 24)) return fail(PKM_EINVAL, "dim must be <= 2^24");
  if (n_rows < 1) return fail(PKM_EINVAL, "n_rows must be >= 1");
  if (n_bags < 0 || n_bags > ((int64_t)1 << 31) - 1) return fail(PKM_EINVAL, "n_bags must be in [0, 2^31)");
  if (bag_size < 1) return fail(PKM_EINVAL, "bag_size must be >= 1");
  if (n_bags == 0) return PKM_OK;
  if (!table || !idx || !w || !y) return fail(PKM_EINVAL, "table, idx, w and y must not be NULL");
  if (((uintptr_t)table & 15) != 0) return fail(PKM_EINVAL, "table must be 16-byte aligned");
  const void* tview = nullptr;
  const int rc = pkm_abi::device_view(table, "table", &tview);
  if (rc != PKM_OK) return rc;
  PKM_LAUNCH(pkm::launch_gather(tview, n_rows, dim, dtype, idx, w, n_bags, bag_size, y, 0, (hipStream_t)stream));
  return PKM_OK;
}

int pkm_enable_stage_timing(pkm_handle* h, int32_t max_records) {
  if (!h) return fail(PKM_EINVAL, "handle is NULL");
  if (max_records < 0 || max_records > 1024) return fail(PKM_EINVAL, "max_records must be in [0, 1024]");
  destroy_timing(h);
  if (max_records == 0) return PKM_OK;
  h->ev.assign((size_t)max_records * EV_PER_REC, nullptr);
  h->rec_mask.assign(max_records, 0u);
  for (hipEvent_t& e : h->ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      destroy_timing(h);
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
    hipEvent_t* e = &h->ev[(size_t)slot * EV_PER_REC + stage * 2];
    float t = __builtin_nanf("");  // a stage not recorded in this forward (masked, or no gate)
    if ((h->rec_mask[slot] >> stage) & 1u && (stage != PKM_STAGE_GATE || h->cfg.memory_plus)) {
      PKM_HIP(hipEventSynchronize(e[1]));
      PKM_HIP(hipEventElapsedTime(&t, e[0], e[1]));
    }
    ms[i] = t;
  }
  return have;
}

int pkm_set_stage_timing_mask(pkm_handle* h, uint32_t mask) {
  if (!h) return fail(PKM_EINVAL, "handle is NULL");
  if (mask >> PKM_NUM_STAGES) return fail(PKM_EINVAL, "mask has bits above stage %d", PKM_NUM_STAGES - 1);
  h->stage_mask = mask;
  return PKM_OK;
}

int pkm_set_score_bound(pkm_handle* h, int32_t mode) {
  if (!h) return fail(PKM_EINVAL, "handle is NULL");
  if (mode != PKM_BOUND_AUTO && mode != PKM_BOUND_EXACT) return fail(PKM_EINVAL, "mode must be PKM_BOUND_AUTO or PKM_BOUND_EXACT");
  h->fp8 = mode == PKM_BOUND_AUTO && pkm::fp8_bound(&h->cfg);
  return PKM_OK;
}

int pkm_destroy(pkm_handle* h) {
  if (!h) return fail(PKM_EINVAL, "handle is NULL");
  destroy_timing(h);
  delete h;
  return PKM_OK;
}

}  // extern "C"
