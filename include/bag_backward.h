/*
 * bag_backward.h -- C ABI of the weighted EmbeddingBag backward and the sparse update
 * on AMD Instinct MI355X (gfx950).
 *
 * The operation, from the forward y[b] = sum over j of w[b, j] * table[idx[b, j]]
 * ("Memory Layers at Scale" digest, parallel EmbeddingBag) by the chain rule, with
 * dy = dL/dy:
 *   dw[b, j]  = <dy[b], table[idx[b, j]]>                                  (fp32)
 *   grad(r)   = sum over (b, j) with idx[b, j] = r of w[b, j] * dy[b]      (fp32)
 *   ds[b, j]  = w[b, j] * (dw[b, j] - sum over the group of w * dw), when w is a
 *               softmax of scores over consecutive groups of `softmax_group` entries
 *               (digest, core idea: the weights are a softmax of the top-k scores)
 *   update    : table[r] = table[r] - lr * grad(r) for every touched row r, rounded
 *               to the table's type: training edits only the slots it read ("Memory
 *               inside the model" overview, learning without forgetting)
 * An index outside [0, n_rows) read nothing and receives nothing (dw = 0).
 *
 * Deterministic: the (row, position) pairs are sorted by row with a stable radix sort
 * and every row's gradient is summed in position order; no atomics.  dw and ds always
 * use the table as it was before the call, also when the update is applied in the same
 * call (dw then comes from the rows the update reads, before they are written).
 *
 * Conventions as in pkm.h (caller-owned DEVICE pointers unless stated, row-major,
 * `stream` a hipStream_t as void*, nothing allocated, PKM_OK or a negative code with
 * the reason in pkm_last_error()).  Not for HIP graph capture: the sort enqueues
 * buffer fills.
 */
#ifndef BAG_BACKWARD_H
#define BAG_BACKWARD_H

#include <stddef.h>
#include <stdint.h>

#include "pkm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  void* table;            /* [n_rows, dim] dtype; device or pinned host memory; written only if update */
  int64_t n_rows;         /* >= 1, < 2^31 */
  int32_t dim;            /* dim * sizeof(dtype) a multiple of 16; dim <= 2048 */
  int32_t dtype;          /* pkm_dtype of the table */
  const int32_t* idx;     /* [n_bags, bag_size] */
  const float* w;         /* [n_bags, bag_size] */
  const float* dy;        /* [n_bags, dim] fp32, 16-byte aligned */
  int64_t n_bags;         /* < 2^24, and n_bags * bag_size < 2^31 */
  int32_t bag_size;       /* 1 .. 2048 */
  float* dw;              /* [n_bags, bag_size] or NULL */
  float* ds;              /* [n_bags, bag_size] or NULL (needs the weights to be a group softmax) */
  int32_t softmax_group;  /* group size of ds, dividing bag_size (ignored when ds is NULL) */
  int32_t* rows;          /* [n_bags * bag_size] or NULL: the distinct rows touched, ascending */
  float* grad;            /* [n_bags * bag_size, dim] or NULL: grad(rows[u]) in row u */
  int32_t* n_unique;      /* device int32 or NULL: the number of distinct rows */
  int32_t update;         /* 1: apply the update with rate lr; 0: leave the table alone */
  float lr;
} pkm_bag_backward_args;

/* Workspace bytes pkm_bag_backward needs for these sizes (sort buffers and temporary
 * storage, 0 if nothing but dw/ds is asked for).  Queries the current device; returns
 * 0 and sets pkm_last_error() on bad sizes. */
size_t pkm_bag_backward_workspace_size(int64_t n_bags, int32_t bag_size, int64_t n_rows);

/* Enqueue the backward on `stream`: without the update, dw and ds from their own pass
 * over the rows; the sort when rows, grad, n_unique or the update are asked for; with
 * the update, one pass per token that updates every touched row once and takes dw from
 * the old rows on the way, then ds; the distinct rows and gradients last.  The workspace
 * (device, 256-byte aligned, ws_bytes >= the size above) is used exclusively by this
 * call until the stream reaches its end. */
int pkm_bag_backward(const pkm_bag_backward_args* args, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of the fixed sort buffers pkm_bag_backward_noalloc uses: enough for 2^21 entries
 * (n_bags * bag_size; e.g. 16,384 tokens x 4 heads x k = 32) over any table. */
#define PKM_BAG_BACKWARD_NOALLOC_BYTES ((size_t)96 << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving or training loops, harnesses that forbid hipMalloc): pkm_bag_backward without a
 * workspace argument.  Its sort buffers are a fixed device array of
 * PKM_BAG_BACKWARD_NOALLOC_BYTES that the library holds on every GPU it runs on until the
 * process ends; the call itself allocates nothing.  Sizes whose
 * pkm_bag_backward_workspace_size exceeds that array are refused with PKM_EWORKSPACE before
 * anything is enqueued (pkm_bag_backward with a caller workspace takes any size).  Results
 * are bitwise those of pkm_bag_backward.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (on different streams or from different threads) race, so
 * the caller orders them (e.g. one stream per GPU). */
int pkm_bag_backward_noalloc(const pkm_bag_backward_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BAG_BACKWARD_H */
