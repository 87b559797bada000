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

constexpr int MAX_CHUNKS = 8;

struct pkm_handle {
  pkm_config cfg;
  int d_h = 0;
  const void* values = nullptr;
  uint8_t* ws = nullptr;
  pkm::Layout L;
  int chunks = 0;  // 0 = automatic
  // pipelining: stream A runs the matrix-core work (selection a1-a6 of every chunk and
  // the gate a8), stream B the gathers (a7); both fork from and join back to the
  // caller's stream
  hipStream_t sA = nullptr, sB = nullptr;
  hipEvent_t ev_fork = nullptr, ev_joinA = nullptr, ev_joinB = nullptr;
  hipEvent_t ev_sel[MAX_CHUNKS] = {};
  hipEvent_t ev_gat[MAX_CHUNKS] = {};
  // stage timing: max_rec records, each with (begin, end) events per stage and chunk plus
  // the whole forward
  int max_rec = 0, next = 0, count = 0;
  uint32_t stage_mask = 0xFFu;  // bit s: stage s is recorded (bit PKM_STAGE_TOTAL: the whole forward)
  std::vector<uint32_t> rec_mask;  // the mask each record was taken with
  std::vector<hipEvent_t> ev;
  std::vector<int> rec_chunks;

  template <typename T = void>
  T* at(size_t off) const { return (T*)(ws + off); }
};

namespace {

constexpr int EV_PER_REC = 7 * MAX_CHUNKS * 2 + 2;

void destroy_timing(pkm_handle* h) {
  for (hipEvent_t e : h->ev)
    if (e) (void)hipEventDestroy(e);
  h->ev.clear();
  h->rec_chunks.clear();
  h->rec_mask.clear();
  h->max_rec = h->next = h->count = 0;
}

void destroy_pipeline(pkm_handle* h) {
  for (hipEvent_t* e : {&h->ev_fork, &h->ev_joinA, &h->ev_joinB})
    if (*e) (void)hipEventDestroy(*e), *e = nullptr;
  for (hipEvent_t& e : h->ev_sel)
    if (e) (void)hipEventDestroy(e), e = nullptr;
  for (hipEvent_t& e : h->ev_gat)
    if (e) (void)hipEventDestroy(e), e = nullptr;
  if (h->sA) (void)hipStreamDestroy(h->sA), h->sA = nullptr;
  if (h->sB) (void)hipStreamDestroy(h->sB), h->sB = nullptr;
}

int create_pipeline(pkm_handle* h) {
  PKM_HIP(hipStreamCreateWithFlags(&h->sA, hipStreamNonBlocking));
  PKM_HIP(hipStreamCreateWithFlags(&h->sB, hipStreamNonBlocking));
  for (hipEvent_t* e : {&h->ev_fork, &h->ev_joinA, &h->ev_joinB}) PKM_HIP(hipEventCreateWithFlags(e, hipEventDisableTiming));
  for (hipEvent_t& e : h->ev_sel) PKM_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  for (hipEvent_t& e : h->ev_gat) PKM_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  return PKM_OK;
}

// Number of token chunks a forward of T tokens is pipelined over.  Measured on MI355X,
// running the gather beside the matrix-core kernels slows both about as much as it
// overlaps them, so the default is one chunk (every stage in order on one stream).
int chunks_for(const pkm_handle* h, int64_t T) {
  if (h->chunks > 0) return (int)(T < h->chunks ? (T > 0 ? T : 1) : h->chunks);
  return 1;
}

struct Timer {
  pkm_handle* h;
  int slot;
  Timer(pkm_handle* h_, int nch) : h(h_), slot(h_->max_rec ? h_->next : -1) {
    if (slot >= 0) {
      h->rec_chunks[slot] = nch;
      h->rec_mask[slot] = h->stage_mask;
    }
  }
  hipEvent_t* base() const { return &h->ev[(size_t)slot * EV_PER_REC]; }
  hipError_t stage(int st, int chunk, int end, hipStream_t s) {
    if (slot < 0 || !((h->rec_mask[slot] >> st) & 1u)) return hipSuccess;
    return hipEventRecord(base()[(st * MAX_CHUNKS + chunk) * 2 + end], s);
  }
  hipError_t total(int end, hipStream_t s) {
    if (slot < 0 || !((h->rec_mask[slot] >> PKM_STAGE_TOTAL) & 1u)) return hipSuccess;
    return hipEventRecord(base()[7 * MAX_CHUNKS * 2 + end], s);
  }
  void commit() {
    if (slot < 0) return;
    h->next = (h->next + 1) % h->max_rec;
    if (h->count < h->max_rec) ++h->count;
  }
};

// Selection scratch of the rows of tokens [t0, ...): group maxima, bounds, candidates.
struct SelScratch {
  float* gmax;
  float* theta;
  uint64_t* cand;
  int32_t* count;
};

SelScratch scratch_at(pkm_handle* h, int64_t t0) {
  const pkm::Layout& L = h->L;
  const size_t r0 = (size_t)t0 * h->cfg.n_heads * 2;  // first row (token, head, half)
  return {h->at<float>(L.gmax) + r0 * pkm::MAX_GROUPS, h->at<float>(L.theta) + r0,
          h->at<uint64_t>(L.cand) + r0 * pkm::CAND, h->at<int32_t>(L.count) + 2 * r0};
}

int run_select(pkm_handle* h, const void* qhat, int64_t T, const SelScratch& sx, int32_t* hidx, float* hsc,
               int32_t* idx, float* sc, float* w, hipStream_t s, Timer* tm, int chunk) {
  const pkm_config& c = h->cfg;
  if (tm) PKM_LAUNCH(tm->stage(PKM_STAGE_SCORE, chunk, 0, s));
  PKM_LAUNCH(pkm::launch_score_candidates(qhat, h->at(h->L.khat), T, c.n_heads, h->d_h, c.n_sub, c.k, c.dtype,
                                          sx.gmax, sx.theta, sx.cand, sx.count, s));
  if (tm) PKM_LAUNCH(tm->stage(PKM_STAGE_SCORE, chunk, 1, s));
  if (tm) PKM_LAUNCH(tm->stage(PKM_STAGE_COMBINE, chunk, 0, s));
  PKM_LAUNCH(pkm::launch_combine(sx.cand, sx.count, T, c.n_heads, c.n_sub, c.k, hidx, hsc, idx, sc, w, s));
  if (tm) PKM_LAUNCH(tm->stage(PKM_STAGE_COMBINE, chunk, 1, s));
  return PKM_OK;
}

// Selection (a1-a6) for tokens [t0, t0 + tc) on stream sa.  The per-half lists are
// written only when `halves` (a debug forward that asks for them): the forward itself needs
// only the final lists.
int chunk_select(pkm_handle* h, const void* x, int64_t t0, int64_t tc, hipStream_t sa, Timer& tm, int chunk,
                 bool halves) {
  const pkm_config& c = h->cfg;
  const pkm::Layout& L = h->L;
  const int H = c.n_heads, dq = c.d_query, k = c.k;
  const size_t eb = c.dtype == PKM_BF16 ? 2 : 4;
  const uint8_t* xc = (const uint8_t*)x + (size_t)t0 * c.d_model * eb;
  float* q = h->at<float>(L.q) + (size_t)t0 * L.qz_cols;
  uint8_t* qhat = h->at<uint8_t>(L.qhat) + (size_t)t0 * H * dq * eb;
  // a1: q = x W_q (fp32); with the Memory+ gate the same GEMM also computes z = x W1 (the
  // first product of a8) into the next d_v columns: one 16,384 x 4,096 product runs
  // faster than two of 16,384 x 2,048 on MI355X
  PKM_LAUNCH(tm.stage(PKM_STAGE_PROJECT, chunk, 0, sa));
  PKM_LAUNCH(pkm::launch_gemm(xc, h->at(L.wqT), q, tc, (int)L.qz_cols, c.d_model, c.dtype, pkm::EPI_STORE_F32, sa));
  PKM_LAUNCH(tm.stage(PKM_STAGE_PROJECT, chunk, 1, sa));
  // a2: qk-norm over each head's d_q, stored in dtype; the halves are the two contiguous halves
  PKM_LAUNCH(tm.stage(PKM_STAGE_QNORM, chunk, 0, sa));
  PKM_LAUNCH(pkm::launch_rownorm(q, 1, qhat, c.dtype, tc * H, dq, c.qk_norm, c.norm_eps, sa, H, L.qz_cols));
  PKM_LAUNCH(tm.stage(PKM_STAGE_QNORM, chunk, 1, sa));
  // a3-a6: scoring + per-half top-k, combine + final top-k + softmax
  const size_t sel = (size_t)t0 * H * k;
  int rc = run_select(h, qhat, tc, scratch_at(h, t0), halves ? h->at<int32_t>(L.hidx) + 2 * sel : nullptr,
                      halves ? h->at<float>(L.hsc) + 2 * sel : nullptr, h->at<int32_t>(L.idx) + sel,
                      h->at<float>(L.sc) + sel, h->at<float>(L.w) + sel, sa, &tm, chunk);
  if (rc || !c.memory_plus) return rc;
  // z = x W1 came with the projection: the stage is kept, empty, so that stage records
  // keep their shape
  PKM_LAUNCH(tm.stage(PKM_STAGE_GATE1, chunk, 0, sa));
  PKM_LAUNCH(tm.stage(PKM_STAGE_GATE1, chunk, 1, sa));
  return PKM_OK;
}

// Gather (a7) for tokens [t0, t0 + tc) on stream sb: with the gate, fused with its
// elementwise part into g = y * silu(z) (dtype); else straight into out.  A debug y
// (fp32) comes from one more plain gather, whose arithmetic is the fused one's.
int chunk_gather(pkm_handle* h, int64_t t0, int64_t tc, void* out, float* ydbg, hipStream_t sb, Timer& tm,
                 int chunk, bool shared) {
  const pkm_config& c = h->cfg;
  const pkm::Layout& L = h->L;
  const int H = c.n_heads, k = c.k;
  const size_t eb = c.dtype == PKM_BF16 ? 2 : 4;
  const int64_t N = (int64_t)c.n_sub * c.n_sub;
  const size_t sel = (size_t)t0 * H * k;
  const int32_t* idx = h->at<int32_t>(L.idx) + sel;
  const float* w = h->at<float>(L.w) + sel;
  PKM_LAUNCH(tm.stage(PKM_STAGE_GATHER, chunk, 0, sb));
  if (c.memory_plus) {
    const float* z = h->at<float>(L.q) + (size_t)t0 * L.qz_cols + (size_t)H * c.d_query;  // columns of x W1
    uint8_t* g = h->at<uint8_t>(L.g) + (size_t)t0 * c.d_value * eb;
    PKM_LAUNCH(pkm::launch_gather(h->values, N, c.d_value, c.dtype, idx, w, tc, H * k, g, 1, sb, z, shared, L.qz_cols));
    if (ydbg)
      PKM_LAUNCH(pkm::launch_gather(h->values, N, c.d_value, c.dtype, idx, w, tc, H * k,
                                    ydbg + (size_t)t0 * c.d_value, 0, sb, nullptr, shared));
  } else {
    uint8_t* o = (uint8_t*)out + (size_t)t0 * c.d_value * eb;
    if (ydbg) {
      float* y = ydbg + (size_t)t0 * c.d_value;
      PKM_LAUNCH(pkm::launch_gather(h->values, N, c.d_value, c.dtype, idx, w, tc, H * k, y, 0, sb, nullptr, shared));
      PKM_LAUNCH(pkm::launch_convert_f32(y, o, tc * c.d_value, c.dtype, sb));
    } else {
      PKM_LAUNCH(pkm::launch_gather(h->values, N, c.d_value, c.dtype, idx, w, tc, H * k, o, 1, sb, nullptr, shared));
    }
  }
  PKM_LAUNCH(tm.stage(PKM_STAGE_GATHER, chunk, 1, sb));
  return PKM_OK;
}

// Memory+ gate (a8), second product, for tokens [t0, t0 + tc) on stream sa: out = g W2.
int chunk_gate(pkm_handle* h, int64_t t0, int64_t tc, void* out, hipStream_t sa, Timer& tm, int chunk) {
  const pkm_config& c = h->cfg;
  const pkm::Layout& L = h->L;
  const size_t eb = c.dtype == PKM_BF16 ? 2 : 4;
  const uint8_t* g = h->at<uint8_t>(L.g) + (size_t)t0 * c.d_value * eb;
  uint8_t* o = (uint8_t*)out + (size_t)t0 * c.d_model * eb;
  PKM_LAUNCH(tm.stage(PKM_STAGE_GATE2, chunk, 0, sa));
  PKM_LAUNCH(pkm::launch_gemm(g, h->at(L.w2T), o, tc, c.d_model, c.d_value, c.dtype,
                              c.dtype == PKM_BF16 ? pkm::EPI_STORE_DT : pkm::EPI_STORE_F32, sa));
  PKM_LAUNCH(tm.stage(PKM_STAGE_GATE2, chunk, 1, sa));
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
  float* ydbg = dbg ? dbg->y : nullptr;
  const bool halves = dbg && (dbg->half_idx || dbg->half_score);

  const int nch = chunks_for(h, T);
  const int64_t tcs = (T + nch - 1) / nch;
  Timer tm(h, nch);
  PKM_LAUNCH(tm.total(0, s));
  const bool gated = c.memory_plus != 0;
  if (nch == 1) {
    int rc = chunk_select(h, x, 0, T, s, tm, 0, halves);
    if (!rc) rc = chunk_gather(h, 0, T, out, ydbg, s, tm, 0, false);
    if (!rc && gated) rc = chunk_gate(h, 0, T, out, s, tm, 0);
    if (rc) return rc;
  } else {
    // fork: both internal streams start after the work already queued on `s`.
    // Stream A: select(0), select(1), gate(0), select(2), gate(1), ...; stream B:
    // gather(c) as soon as select(c) is done.  So the gather of one chunk runs beside
    // the matrix-core work of its neighbours.
    PKM_HIP(hipEventRecord(h->ev_fork, s));
    PKM_HIP(hipStreamWaitEvent(h->sA, h->ev_fork, 0));
    PKM_HIP(hipStreamWaitEvent(h->sB, h->ev_fork, 0));
    auto span = [&](int ch, int64_t& t0, int64_t& tc) {
      t0 = ch * tcs;
      tc = T - t0 < tcs ? T - t0 : tcs;
    };
    int last = -1;
    for (int ch = 0; ch < nch; ++ch) {
      int64_t t0, tc;
      span(ch, t0, tc);
      if (tc <= 0) break;
      int rc = chunk_select(h, x, t0, tc, h->sA, tm, ch, halves);
      if (rc) return rc;
      PKM_HIP(hipEventRecord(h->ev_sel[ch], h->sA));
      PKM_HIP(hipStreamWaitEvent(h->sB, h->ev_sel[ch], 0));
      rc = chunk_gather(h, t0, tc, out, ydbg, h->sB, tm, ch, true);
      if (rc) return rc;
      PKM_HIP(hipEventRecord(h->ev_gat[ch], h->sB));
      if (gated && ch > 0) {
        int64_t p0, pc;
        span(ch - 1, p0, pc);
        PKM_HIP(hipStreamWaitEvent(h->sA, h->ev_gat[ch - 1], 0));
        rc = chunk_gate(h, p0, pc, out, h->sA, tm, ch - 1);
        if (rc) return rc;
      }
      last = ch;
    }
    if (gated && last >= 0) {
      int64_t p0, pc;
      span(last, p0, pc);
      PKM_HIP(hipStreamWaitEvent(h->sA, h->ev_gat[last], 0));
      int rc = chunk_gate(h, p0, pc, out, h->sA, tm, last);
      if (rc) return rc;
    }
    // join: `s` continues after both internal streams
    PKM_HIP(hipEventRecord(h->ev_joinA, h->sA));
    PKM_HIP(hipEventRecord(h->ev_joinB, h->sB));
    PKM_HIP(hipStreamWaitEvent(s, h->ev_joinA, 0));
    PKM_HIP(hipStreamWaitEvent(s, h->ev_joinB, 0));
  }
  PKM_LAUNCH(tm.total(1, s));
  tm.commit();

  int32_t* idx = h->at<int32_t>(L.idx);
  float* w = h->at<float>(L.w);
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

const char* pkm_last_error(void) { return pkm_abi::last_error(); }

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
    destroy_pipeline(h);
    delete h;
    return code;
  };
  rc = create_pipeline(h);
  if (rc) {
    destroy_pipeline(h);
    return bail(rc);
  }
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
  return run_select(h, qhat, T, scratch_at(h, 0), half_idx ? half_idx : h->at<int32_t>(L.hidx), half_score ? half_score : h->at<float>(L.hsc),
                    idx ? idx : h->at<int32_t>(L.idx), score ? score : h->at<float>(L.sc), w ? w : h->at<float>(L.w),
                    (hipStream_t)stream, nullptr, 0);
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
  h->rec_chunks.assign(max_records, 0);
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
  const bool gated = h->cfg.memory_plus != 0;
  for (int i = 0; i < have; ++i) {
    const int slot = (first + skip + i) % h->max_rec;
    hipEvent_t* e = &h->ev[(size_t)slot * EV_PER_REC];
    float sum = 0.f;
    if (!((h->rec_mask[slot] >> stage) & 1u)) {
      sum = __builtin_nanf("");  // not recorded in this forward
    } else if (stage == PKM_STAGE_TOTAL) {
      PKM_HIP(hipEventSynchronize(e[7 * MAX_CHUNKS * 2 + 1]));
      PKM_HIP(hipEventElapsedTime(&sum, e[7 * MAX_CHUNKS * 2], e[7 * MAX_CHUNKS * 2 + 1]));
    } else if (gated || (stage != PKM_STAGE_GATE1 && stage != PKM_STAGE_GATE2)) {
      // sum over the chunks: the time this stage's kernels spent, each measured on its stream
      for (int c = 0; c < h->rec_chunks[slot]; ++c) {
        float t = 0.f;
        PKM_HIP(hipEventSynchronize(e[(stage * MAX_CHUNKS + c) * 2 + 1]));
        PKM_HIP(hipEventElapsedTime(&t, e[(stage * MAX_CHUNKS + c) * 2], e[(stage * MAX_CHUNKS + c) * 2 + 1]));
        sum += t;
      }
    }
    ms[i] = sum;
  }
  return have;
}

int pkm_set_stage_timing_mask(pkm_handle* h, uint32_t mask) {
  if (!h) return fail(PKM_EINVAL, "handle is NULL");
  if (mask >> PKM_NUM_STAGES) return fail(PKM_EINVAL, "mask has bits above stage %d", PKM_NUM_STAGES - 1);
  h->stage_mask = mask;
  return PKM_OK;
}

int pkm_set_pipeline_chunks(pkm_handle* h, int32_t chunks) {
  if (!h) return fail(PKM_EINVAL, "handle is NULL");
  if (chunks < 0 || chunks > MAX_CHUNKS) return fail(PKM_EINVAL, "chunks must be in [0, %d]", MAX_CHUNKS);
  h->chunks = chunks;
  return PKM_OK;
}

int pkm_destroy(pkm_handle* h) {
  if (!h) return fail(PKM_EINVAL, "handle is NULL");
  destroy_timing(h);
  destroy_pipeline(h);
  delete h;
  return PKM_OK;
}

}  // extern "C"
