/*
 * engram.h -- C ABI of the hashed n-gram lookup (Engram) on AMD Instinct MI355X (gfx950).
 *
 * The operation (review of "Conditional Memory via Scalable Lookup" (Engram), cited by
 * section and equation):
 *  - sparse retrieval, multi-head hashing, key equation 1: the n-grams ending at a
 *    token are hashed by several independent hash functions phi_{n,k} into the rows
 *    of per-(order, head) embedding tables, e_{t,n,k} = E_{n,k}[phi_{n,k}(g_{t,n})];
 *  - sparse retrieval, tokenizer compression: ids with one meaning share one id
 *    (an optional vocabulary map);
 *  - context-aware fusion, gating, key equation 2:
 *    alpha_t = sigmoid(RMSNorm(h_t) . RMSNorm(e_t) / sqrt(d));
 *  - context-aware fusion, residual connection: the result is added to h_t.
 *
 * What engram_forward computes for every token t (orders n = min_order + o,
 * o < n_orders; heads k < n_heads; P = table_rows; d = n_heads * head_dim):
 *   id'_j      = compress[id_j] if compress else id_j, with any id_j outside
 *                [0, vocab) read as 0
 *   g_{t,n}    = (id'_{t-n+1}, ..., id'_t), positions before the start of t's
 *                sequence (sequences are seq_len consecutive tokens) read as id 0
 *   phi_{n,k}  = fold over g, oldest first, of h <- ((h XOR id) * mult[o][k]) mod 2^64
 *                from h = 0, then h mod P
 *   row_{t,k,o} = (o * n_heads + k) * P + phi_{n,k}(g_{t,n})   (row of the stacked table)
 *   e_t[k * head_dim + i] = sum over o of tables[row_{t,k,o}][i]          (fp32)
 *   alpha_t    = 1 / (1 + exp(-z)), z = <h_t, e_t> / (sqrt(mean(h_t^2) + eps)
 *                * sqrt(mean(e_t^2) + eps) * sqrt(d))                     (fp32)
 *   out_t      = alpha_t * e_t  (+ h_t if residual), stored in dtype (RNE for bf16)
 *
 * Conventions (as in pkm.h): tensor pointers are caller-owned DEVICE pointers,
 * row-major; `stream` is a hipStream_t as void* (NULL = default stream); the calls
 * only enqueue work, allocate nothing and never wait for the GPU (engram_forward can
 * be captured in a HIP graph); the return is PKM_OK or a negative PKM_E* code with the
 * reason in pkm_last_error().
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stdint.h>

#include "pkm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t min_order;  /* smallest n-gram order, >= 1 */
  int32_t n_orders;   /* orders min_order .. min_order + n_orders - 1; 1..4, largest <= 8 */
  int32_t n_heads;    /* hash heads (and tables) per order, 1..64 */
  int32_t head_dim;   /* width of one table row; head_dim * sizeof(dtype) a multiple of 16 */
  int64_t table_rows; /* rows P of every table E_{n,k}; n_orders * n_heads * P < 2^31 */
  int32_t vocab;      /* ids outside [0, vocab) read as 0; length of the compress map; >= 1 */
  int32_t dtype;      /* pkm_dtype of the tables, h and out */
  int32_t residual;   /* 0: out = alpha * e; 1: out = h + alpha * e */
  float norm_eps;     /* RMSNorm epsilon, in [0, 1] */
} engram_config;
/* Limits: d = n_heads * head_dim with d * sizeof(dtype) <= 4096 bytes (one wave holds a
 * token's d values, four 16-byte slices per lane); 0 <= T <= 2^25 tokens per call (one wave
 * per token); seq_len >= 1. */

/* Rows of the stacked table for every (token, head, order), per the formulas above.
 *   ids      [T] int32; seq_len >= 1 tokens per sequence (T need not be a multiple)
 *   compress [vocab] int32 ids >= 0, or NULL (identity)
 *   mult     [n_orders, n_heads] uint64 hash multipliers (any values; odd ones make
 *            each fold step a bijection)
 *   rows     [T, n_heads, n_orders] int32 output
 * Integer-exact.  T = 0 is a no-op. */
int engram_hash(const engram_config* cfg, const int32_t* ids, int64_t T, int64_t seq_len, const int32_t* compress,
                const uint64_t* mult, int32_t* rows, void* stream);

/* The whole lookup in one kernel (hash, gather-sum of the n_orders rows per head,
 * gate, output).
 *   tables [n_orders * n_heads * P, head_dim] dtype: E_{n,k} stacked, table
 *          (o * n_heads + k) first; 16-byte aligned; borrowed
 *   h      [T, d] dtype hidden states; out [T, d] dtype
 *   e_out  [T, d] float or NULL: e_t (fp32) for inspection
 *   alpha_out [T] float or NULL: alpha_t
 * T = 0 is a no-op. */
int engram_forward(const engram_config* cfg, const void* tables, const int32_t* ids, int64_t T, int64_t seq_len,
                   const int32_t* compress, const uint64_t* mult, const void* h, void* out, float* e_out,
                   float* alpha_out, void* stream);

/* Host-resident tables with prefetch (review of "Conditional Memory via Scalable
 * Lookup" (Engram): the tables can live in host memory at a small cost in throughput;
 * summary of "Memory Attention", how it is used: the lookup addresses depend only on
 * token ids, so the rows can be fetched before the hidden state that needs them).
 *
 * engram_prefetch computes the rows of every (token, order, head) exactly as
 * engram_forward does and copies them, in their stored type, to
 *   staged [T, n_orders, d] dtype (device memory): staged[t, o, k*head_dim + i] =
 *          tables[row_{t,k,o}][i]
 * `tables` may be device memory or pinned host memory (allocated with hipHostMalloc,
 * or a pinned torch tensor): the kernel then reads it over the host link.  Pageable
 * host memory is refused (PKM_EINVAL).  Launch it early on a side stream and order
 * engram_forward_staged after it with an event.
 *
 * engram_forward_staged computes e_t (the sum over orders of staged[t, o, :]), the gate
 * and the output exactly as engram_forward does (same arithmetic in the same order, so
 * the results are bitwise equal); h, out, e_out, alpha_out as for engram_forward.
 * T = 0 is a no-op for both. */
int engram_prefetch(const engram_config* cfg, const void* tables, const int32_t* ids, int64_t T, int64_t seq_len,
                    const int32_t* compress, const uint64_t* mult, void* staged, void* stream);
int engram_forward_staged(const engram_config* cfg, const void* staged, const void* h, int64_t T, void* out,
                          float* e_out, float* alpha_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */
