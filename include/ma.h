/*
 * ma.h -- C ABI of the Memory Attention token-memory values on AMD Instinct MI355X (gfx950).
 *
 * The operation (summary of "Memory Attention", cited by section):
 *  - how it works: a per-layer table E [vocab, d_v] is read by the input token id s,
 *    an RMSNorm is applied to each token vector within every key/value head (M), and
 *    the attention values are V = K + M, with no value projection;
 *  - how it differs: at inference the norm is folded into the table beforehand,
 *    E_bar[i] = Norm(E[i]), so building the values is one lookup (a k = 1, weight-1
 *    EmbeddingBag) and one elementwise add: V = K + E_bar[s].
 *
 * Conventions as in pkm.h: caller-owned DEVICE pointers, row-major; `stream` is a
 * hipStream_t as void*; the calls only enqueue work and allocate nothing (ma_values
 * can be captured in a HIP graph); the return is PKM_OK or a negative PKM_E* code with
 * the reason in pkm_last_error().
 */
#ifndef MA_H
#define MA_H

#include <stdint.h>

#include "pkm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* E_bar[i, h*hd : (h+1)*hd] = E[i, slice] / sqrt(mean(E[i, slice]^2) + eps) * gain[slice]
 * for every row i < vocab and head h < n_heads (hd = d_v / n_heads), computed in fp32
 * and stored in dtype (RNE for bf16).
 *   E, E_bar [vocab, d_v] dtype (E_bar may equal E: in place); gain [d_v] float or NULL (1)
 *   d_v * sizeof(dtype) a multiple of 16; d_v a multiple of n_heads, and
 *   (d_v / n_heads) * sizeof(dtype) a multiple of 16; eps in [0, 1]; vocab * n_heads <= 2^38. */
int ma_fold_table(const void* E, int64_t vocab, int32_t d_v, int32_t n_heads, const float* gain, float eps,
                  int32_t dtype, void* E_bar, void* stream);

/* V[t] = K[t] + E_bar[ids[t]] for t < T (fp32 add, stored in dtype); an id outside
 * [0, vocab) reads no row (V[t] = K[t]).
 *   E_bar [vocab, d_v], K and V [T, d_v] dtype, 16-byte aligned; ids [T] int32.
 *   vocab >= 1; T * d_v * sizeof(dtype) / 16 <= 2^38.  T = 0 is a no-op. */
int ma_values(const void* E_bar, int64_t vocab, int32_t d_v, int32_t dtype, const int32_t* ids, int64_t T,
              const void* K, void* V, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MA_H */
