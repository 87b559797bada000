/*
 * pkm.h -- C ABI of the product-key memory forward on AMD Instinct MI355X (gfx950).
 *
 * The operation (cited by page title and section):
 *  - "Memory Layers at Scale" digest, core idea: a memory layer holds trainable
 *    key/value pairs, picks the top-k keys most similar to the input token and
 *    returns the weighted sum of their values, in place of an FFN.
 *  - same page, product-key search: every key is split into two sub-keys, so the
 *    top-k is found with 2*sqrt(N) comparisons instead of N.
 *  - "Memory inside the model" overview, how it works: the query is split into
 *    a front and a back half, each half is compared with its own list of
 *    half-keys, and the best of both lists are combined; about thirty values
 *    are read and averaged with weights; a gate decides how much goes on.
 *  - digest, Memory+ block: out = (y * silu(x W1)) W2, with qk-normalisation.
 *  - digest, parallel EmbeddingBag: the value read is a weighted EmbeddingBag
 *    and is bound by memory bandwidth.
 *
 * What pkm_forward computes for every token t (row-major, per head h < H):
 *   q        = x[t] W_q[:, h*d_q : (h+1)*d_q]           (fp32 accumulate, stored in dtype)
 *   qhat     = RMSNorm(q) if qk_norm else q, over all d_q; stored in dtype
 *   s_c[i]   = <qhat[c*d_h : (c+1)*d_h], Khat[h, c, i]>, c in {0, 1}, i < n_sub
 *              where Khat = RMSNorm(subkeys) per row if qk_norm (folded at create)
 *   top-k of each half under (score desc, index asc)
 *   cells    = the k*k pairs (a, b): score s_0[a] + s_1[b] (fp32), flat index a*n_sub + b
 *   idx, sc  = top-k cells under (score desc, flat index asc)
 *   w        = softmax(sc)                                             (per head)
 *   y[t]     = sum over h, j of w[h, j] * V[idx[h, j]]                 (fp32 accumulate)
 *   out[t]   = memory_plus ? (y * silu(z)) W2 : y, z = x[t] W1 (stored in dtype)
 * With dtype = BF16, q, z, qhat, Khat and y * silu(z) are rounded to bf16
 * (round-to-nearest-even): a bf16 product returns q and z in bf16, and the norm and
 * the gate read those stored values; scores, softmax and y are fp32.
 *
 * Conventions for every call below:
 *  - Pointers to tensors are DEVICE pointers, row-major, owned by the caller
 *    (typically PyTorch tensors) and must stay valid while in use.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work and returns without waiting for the GPU;
 *    the forward allocates nothing and performs no host sync, so a forward can
 *    be captured in a HIP graph and replayed once an earlier call with the same
 *    number of tokens has made its GEMM plans (bf16: host work only; the first
 *    call whose token count falls in a new power-of-two bucket also runs one
 *    hipBLASLt heuristic query, about 0.1 s).  Its results are ordered on
 *    `stream`: work enqueued on `stream` afterwards sees them.
 *  - A handle belongs to the device that is current at pkm_create.  One call at
 *    a time may use a handle; different handles may be used by different host
 *    threads at once (the library's shared GEMM plans are guarded by a lock).
 *  - Return value: PKM_OK (0) or a negative PKM_E* code; on error, the message
 *    is available from pkm_last_error() (thread-local) and nothing was enqueued
 *    unless the code is PKM_EHIP.  Nothing aborts and no C++ exception leaves
 *    the library.  Faults of kernels already enqueued surface at the caller's
 *    next synchronisation.
 */
#ifndef PKM_H
#define PKM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PKM_OK = 0,
  PKM_EINVAL = -1,        /* bad argument or shape */
  PKM_EUNSUPPORTED = -2,  /* device is not gfx950, or a valid shape outside the built kernels (d_query > 512) */
  PKM_EWORKSPACE = -3,    /* workspace too small */
  PKM_EHIP = -4           /* a HIP runtime call failed (message has the HIP error) */
};

typedef enum { PKM_F32 = 0, PKM_BF16 = 1 } pkm_dtype;

typedef struct {
  int32_t d_model;      /* width of x, <= 65536; a multiple of 32 for bf16 (4 for fp32) */
  int32_t n_heads;      /* 1 <= H <= 64 */
  int32_t d_query;      /* per-head query width d_q: even, 2..512 (larger: PKM_EUNSUPPORTED) */
  int32_t n_sub;        /* sub-keys per half; the table has N = n_sub^2 < 2^31 rows */
  int32_t k;            /* per-half and final top-k, 1 <= k <= min(n_sub, 64) */
  int32_t d_value;      /* value width, <= 65536; d_value * sizeof(dtype) a multiple of 16 (bf16 Memory+: of 64) */
  int32_t dtype;        /* pkm_dtype of x, W_q, subkeys, values, W1, W2 and out */
  int32_t qk_norm;      /* 0 or 1: RMSNorm of the query (before the split) and of sub-key rows */
  int32_t memory_plus;  /* 0: out = y [T, d_value]; 1: gated out [T, d_model] */
  float norm_eps;       /* RMSNorm epsilon in [0, 1] (1e-6 in the shipped workloads) */
  int64_t max_tokens;   /* largest T a forward may take, 1..2^24 with max_tokens * n_heads <= 2^24;
                           sizes the workspace */
} pkm_config;

/* Stage ids for the optional per-stage timing. */
enum {
  PKM_STAGE_PROJECT = 0,  /* q = x W_q (Memory+: with z = x W1 in the same GEMM) */
  PKM_STAGE_QNORM = 1,    /* qk-norm + split */
  PKM_STAGE_SCORE = 2,    /* sub-key scoring fused with the per-half top-k */
  PKM_STAGE_COMBINE = 3,  /* k x k combine, final top-k, softmax */
  PKM_STAGE_GATHER = 4,   /* weighted EmbeddingBag over the value table (Memory+: with y * silu(z)) */
  PKM_STAGE_GATE = 5,     /* (y * silu(z)) W2 (Memory+ only; z = x W1 comes with the projection) */
  PKM_STAGE_TOTAL = 6,    /* the whole forward */
  PKM_NUM_STAGES = 7
};

typedef struct pkm_handle pkm_handle; /* opaque */

/* Optional intermediate outputs of pkm_forward_debug; every pointer may be NULL.
 *   qhat       [T, H, 2, d_h] dtype   normalised query halves as scored
 *   half_idx   [T, H, 2, k]  int32    per-half top-k sub-key indices, best first
 *   half_score [T, H, 2, k]  fp32     their scores
 *   idx        [T, H, k]     int32    final flat indices a*n_sub + b, best first
 *   score      [T, H, k]     fp32     final scores
 *   w          [T, H, k]     fp32     softmax weights
 *   y          [T, d_value]  fp32     gathered values before the gate
 *   theta      [T, H, 2]     fp32     the per-half selection bound of the two scoring passes
 *                                     (unspecified when every row is scored exhaustively:
 *                                     fewer than 2k groups of sub-keys, k + 32 for k > 32)
 *   counts     [T, H, 2, 2]  int32    candidates per lane half after the overflow pass
 *                                     (same condition)                                    */
typedef struct {
  void* qhat;
  int32_t* half_idx;
  float* half_score;
  int32_t* idx;
  float* score;
  float* w;
  float* y;
  float* theta;
  int32_t* counts;
} pkm_debug_ptrs;

/* Bytes of device workspace a handle with this config needs (0 if the config is
 * invalid; see pkm_last_error).  The workspace holds the repacked weights, the
 * normalised sub-keys and every per-forward intermediate for max_tokens tokens. */
size_t pkm_workspace_size(const pkm_config* cfg);

/* Create a handle.  Enqueues on `stream`: the repacking of W_q (and W1, W2) into
 * the workspace and the fold of the sub-key RMSNorm into a normalised copy
 * (the handle therefore snapshots W_q, subkeys, W1, W2 as they are when the
 * stream reaches this work).  `values` is borrowed, not copied: it must stay
 * valid and unchanged while the handle is used.
 *   W_q      [d_model, H*d_q]   (head h = columns h*d_q .. h*d_q + d_q - 1)
 *   subkeys  [H, 2, n_sub, d_h] (index 0 scores the first query half)
 *   values   [n_sub^2, d_value]: device memory, or pinned host memory (hipHostMalloc,
 *            a pinned torch tensor) read by the gather over the host link (a
 *            host-resident table: the roofline becomes the host link's bandwidth);
 *            pageable host memory is refused (PKM_EINVAL)
 *   W1       [d_model, d_value], W2 [d_value, d_model]  (NULL unless memory_plus)
 *   workspace: device buffer of ws_bytes >= pkm_workspace_size(cfg), 256-byte
 *            aligned, owned by the caller, used exclusively by this handle.
 * W_q, subkeys, W1, W2 and the workspace must be device memory (checked).
 * Errors: PKM_EINVAL (bad config, NULL or non-device pointer), PKM_EWORKSPACE,
 * PKM_EUNSUPPORTED (device not gfx950, or d_query > 512), PKM_EHIP. */
int pkm_create(const pkm_config* cfg, const void* W_q, const void* subkeys, const void* values,
               const void* W1, const void* W2, void* workspace, size_t ws_bytes, void* stream,
               pkm_handle** out);

/* The forward for T tokens (0 <= T <= max_tokens; T = 0 enqueues nothing).
 * Every stage runs in order on `stream`.
 *   x        [T, d_model] dtype
 *   out      [T, d_model] dtype if memory_plus, else [T, d_value] dtype
 *   idx_out  [T, H, k] int32, optional (NULL): final flat indices
 *   w_out    [T, H, k] fp32, optional (NULL): softmax weights
 * One forward may be in flight per handle (the workspace is reused). */
int pkm_forward(pkm_handle* h, const void* x, int64_t T, void* out, int32_t* idx_out, float* w_out,
                void* stream);

/* The same forward, also copying the intermediates named in `dbg` (may be NULL). */
int pkm_forward_debug(pkm_handle* h, const void* x, int64_t T, void* out, const pkm_debug_ptrs* dbg,
                      void* stream);

/* Selection only (scoring, per-half top-k, combine, softmax) from a given
 * normalised query qhat [T, H, 2, d_h] in dtype, against the handle's
 * normalised sub-keys.  Outputs as in pkm_debug_ptrs; half_* may be NULL. */
int pkm_select(pkm_handle* h, const void* qhat, int64_t T, int32_t* half_idx, float* half_score,
               int32_t* idx, float* score, float* w, void* stream);

/* Copy the handle's normalised sub-keys [H, 2, n_sub, d_h] (dtype) to `dst`. */
int pkm_copy_normalized_subkeys(pkm_handle* h, void* dst, void* stream);

/* Weighted EmbeddingBag in sum mode over a table of n_rows x dim (dtype):
 *   y[b, :] = sum over j < bag_size of w[b, j] * table[idx[b, j], :]     (fp32)
 * idx [n_bags, bag_size] int32, w [n_bags, bag_size] fp32, y [n_bags, dim] fp32.
 * Indices outside [0, n_rows) contribute nothing.  dim <= 2^24, dim * sizeof(dtype) a
 * multiple of 16 and the table 16-byte aligned; the table may be device memory or
 * pinned host memory (as `values` of pkm_create).  n_bags = 0 enqueues nothing. */
int pkm_embedding_bag(const void* table, int64_t n_rows, int32_t dim, int32_t dtype,
                      const int32_t* idx, const float* w, int64_t n_bags, int32_t bag_size, float* y,
                      void* stream);

/* Per-stage timing with HIP events recorded on the forward's stream around each
 * stage's launches.  pkm_enable_stage_timing keeps the last `max_records` forwards
 * (0 turns it off); it allocates the events, so call it outside any timed or
 * captured region.  pkm_stage_times waits for the recorded events, writes up to `n`
 * durations in milliseconds of stage `stage` (PKM_STAGE_*) for the recorded
 * forwards, oldest first, and returns how many it wrote (or a negative error code).
 * PKM_STAGE_GATE reads NaN for a handle without the Memory+ gate. */
int pkm_enable_stage_timing(pkm_handle* h, int32_t max_records);
int pkm_stage_times(pkm_handle* h, int32_t stage, float* ms, int32_t n);

/* Which stages the following forwards record: bit s (1u << PKM_STAGE_*) set records
 * stage s; the default records all of them.  Every event pair costs the forward a
 * few microseconds, so a run that times whole forwards can keep only the stages it
 * needs.  A stage left out of a recorded forward reads as NaN in pkm_stage_times.
 * Returns PKM_EINVAL for bits at or above PKM_NUM_STAGES. */
int pkm_set_stage_timing_mask(pkm_handle* h, uint32_t mask);

/* How the scoring bounds the k-th best score of every (token, head, half) before it collects
 * candidates.  PKM_BOUND_AUTO (the default): bf16 workloads whose query halves are stored 256
 * wide (d_query / 2 in 129..256) estimate it from the group maxima of fp8 (OCP e4m3) scores
 * lowered by a margin, and every other workload takes PKM_BOUND_EXACT: the group maxima of the
 * scores in the stored type.  The result is the same either way: the candidates are the exact
 * scores at or above the bound, and a row left with fewer than k is scored exhaustively, so
 * the bound only decides how much work the selection does. */
enum { PKM_BOUND_AUTO = 0, PKM_BOUND_EXACT = 1 };
int pkm_set_score_bound(pkm_handle* h, int32_t mode);

/* Release the handle's host state and events (the workspace stays the caller's). */
int pkm_destroy(pkm_handle* h);

/* Message of the last error on this thread ("" if none). */
const char* pkm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKM_H */
