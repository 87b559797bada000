"""Oracle of the product-key memory forward (TEST INFRASTRUCTURE; float64 NumPy).

Sources (cited by page title and section):

* "Memory Layers at Scale" digest -- section "core idea" (a memory layer keeps
  trainable key/value pairs, picks the top-k keys most similar to the input
  token and returns the weighted sum of their values), section "product-key
  search" (each key is split into two sub-keys; top-k is found with 2*sqrt(N)
  comparisons instead of N), section "Memory+ block" (the gated output
  (y * silu(x W1)) W2 and qk-normalisation), section "parallel EmbeddingBag"
  (the value read is an EmbeddingBag).
* "Memory inside the model" overview -- section "how it works" (split the query
  into a front and a back half, compare each half with its list of half-keys,
  combine the best of both, which gives the right answer among all cells; read
  about thirty values and take their weighted average) and Figure D (8 + 8
  comparisons find the best of 64 cells).

Readings of points the pages leave open (each is listed with its reason in the
design notes of the repository):

* heads: H independent query projections and sub-key codebooks over one shared
  value table; each head selects and normalises its own top-k; head outputs are
  summed (the gather is one bag of H*k rows per token).
* qk-norm: RMSNorm v / sqrt(mean(v^2) + eps) with unit gain; the query is
  normalised over its full per-head width before the split; each sub-key row
  is normalised over its own width; no extra score scale.
* flat index of cell (a, b) = a * n_sub + b (the first half is the major index).
* order: score descending, then index ascending (the lowest index wins a tie);
  -0.0 compares equal to +0.0.
* softmax over each head's final k scores, no temperature.
* bf16 workloads: the projections q = x W_q and z = x W1 are stored in bf16 (the
  type a bf16 product returns) before the norm and the gate read them; the
  normalised query and sub-keys are rounded to bf16 before scoring, and
  y * silu(z) is rounded to bf16 before W2; all other arithmetic here is float64
  on the exact stored values.

Arrays of stored bf16 values are uint16 bit patterns; float32 storage is
float32.
"""

from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------------
# stored values <-> float64


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: the bits are the top half of a float32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 values once to bf16 (8 significant bits, round-to-nearest-even).

    A float64 has 52 stored fraction bits and a bf16 keeps 7, so the low 45 bits
    are rounded away; the result is then exact in float32 and its top 16 bits are
    the bf16 pattern.  Finite values in the normal float32 range only.
    """
    u = np.ascontiguousarray(v, dtype=np.float64).view(np.uint64)
    half = np.uint64(1 << 44)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = ((u + (half - np.uint64(1)) + lsb) >> np.uint64(45)) << np.uint64(45)
    f32 = r.view(np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f64(a) if dtype == "bf16" else np.asarray(a, dtype=np.float64)


def round_stored(v: np.ndarray, dtype: str) -> np.ndarray:
    """Value after storage in ``dtype``: bf16 rounding for bf16, identity for f32 math in f64."""
    return bf16_bits_to_f64(f64_to_bf16_bits(v)) if dtype == "bf16" else v


# ----------------------------------------------------------------------------------
# the steps, in the order of the forward


def rmsnorm(v: np.ndarray, eps: float) -> np.ndarray:
    """qk-norm ("Memory Layers at Scale" digest, Memory+ block): RMSNorm over the last axis."""
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)


def project_query(x: np.ndarray, W_q: np.ndarray, H: int, d_q: int) -> np.ndarray:
    """The query of each head ("Memory inside the model" overview, how it works): q = x W_q.

    x [T, d_model], W_q [d_model, H*d_q] -> q [T, H, d_q].
    """
    q = x @ W_q
    return q.reshape(x.shape[0], H, d_q)


def split_halves(q: np.ndarray):
    """Front and back half of the query (overview, how it works)."""
    d_h = q.shape[-1] // 2
    return q[..., :d_h], q[..., d_h:]


def half_scores(q_half: np.ndarray, keys_half: np.ndarray) -> np.ndarray:
    """Scores of one query half against its list of half-keys (digest, product-key search).

    q_half [T, H, d_h], keys_half [H, n, d_h] -> s [T, H, n], s[t,h,i] = <q_half[t,h], keys_half[h,i]>.
    """
    return np.einsum("thd,hnd->thn", q_half, keys_half)


def topk_order(scores: np.ndarray, k: int):
    """Top-k along the last axis under (score descending, index ascending).

    Returns (indices, scores) of shape [..., k], best first.  A stable sort of
    the negated scores with the index as the secondary key gives exactly this
    order; -0.0 and +0.0 compare equal.
    """
    n = scores.shape[-1]
    ar = np.broadcast_to(np.arange(n), scores.shape)
    order = np.lexsort((ar, -scores), axis=-1)[..., :k]
    return order.astype(np.int64), np.take_along_axis(scores, order, axis=-1)


def combine_topk(s1, i1, s2, i2, n_sub: int, k: int):
    """Combine the best of both halves and keep the final top-k (overview, how it works).

    The score of cell (a, b) is the sum of its half scores (the key is the
    concatenation of two sub-keys: digest, product-key search); its flat index
    is a * n_sub + b.  Every pair of the k x k candidates is formed; the final
    top-k is taken under (sum descending, flat index ascending).
    s1, i1, s2, i2: [T, H, k]. Returns (flat [T,H,k], score [T,H,k]).
    """
    sums = s1[..., :, None] + s2[..., None, :]
    flat = i1[..., :, None] * n_sub + i2[..., None, :]
    shp = sums.shape[:-2] + (sums.shape[-2] * sums.shape[-1],)
    sums = sums.reshape(shp)
    flat = flat.reshape(shp)
    order = np.lexsort((flat, -sums), axis=-1)[..., :k]
    return np.take_along_axis(flat, order, axis=-1), np.take_along_axis(sums, order, axis=-1)


def softmax(s: np.ndarray) -> np.ndarray:
    """Normalised weights of one head's k scores (weighted sum/average: digest core idea,
    overview how it works); max-subtracted exponentials over the last axis."""
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def weighted_bag(rows_of, idx: np.ndarray, w: np.ndarray) -> np.ndarray:
    """EmbeddingBag with per-sample weights in sum mode (digest, parallel EmbeddingBag).

    y[t, :] = sum over all (h, j) of w[t, h, j] * V[idx[t, h, j], :].
    ``rows_of(r)`` returns the float64 rows r of V, shape [len(r), d_v].
    A row chosen twice counts twice.
    """
    T = idx.shape[0]
    flat_idx = idx.reshape(T, -1)
    flat_w = w.reshape(T, -1).astype(np.float64)
    y = None
    for t in range(T):
        rows = rows_of(flat_idx[t])
        yt = (flat_w[t][:, None] * rows).sum(axis=0)
        if y is None:
            y = np.empty((T, rows.shape[1]), dtype=np.float64)
        y[t] = yt
    return y


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def memory_plus(y: np.ndarray, x: np.ndarray, W1: np.ndarray, W2: np.ndarray, dtype: str) -> np.ndarray:
    """Memory+ output (digest, Memory+ block): out = (y * silu(x W1)) W2, row-major form.

    For bf16 workloads z = x W1 and the gated product are each stored as bf16 before
    they are used.
    """
    z = round_stored(x @ W1, dtype)
    g = round_stored(y * silu(z), dtype)
    return g @ W2


# ----------------------------------------------------------------------------------
# composite stages


def normalized_query(x, W_q, H, d_q, qk_norm: bool, eps: float, dtype: str):
    """q stored in dtype -> optional RMSNorm over d_q -> rounding to the scoring precision
    -> halves."""
    q = round_stored(project_query(x, W_q, H, d_q), dtype)
    if qk_norm:
        q = rmsnorm(q, eps)
    q = round_stored(q, dtype)
    return split_halves(q)


def normalized_subkeys(subkeys, qk_norm: bool, eps: float, dtype: str):
    """Sub-key codebooks [H, 2, n, d_h] -> (K1 [H,n,d_h], K2 [H,n,d_h]) after optional RMSNorm."""
    K = rmsnorm(subkeys, eps) if qk_norm else subkeys
    K = round_stored(K, dtype)
    return K[:, 0], K[:, 1]


def select(q1, q2, K1, K2, k: int):
    """Stages from scoring to weights for every (token, head).

    Returns a dict: half_idx [T,H,2,k], half_score [T,H,2,k], idx [T,H,k] (flat),
    score [T,H,k], w [T,H,k].
    """
    n_sub = K1.shape[1]
    s1 = half_scores(q1, K1)
    s2 = half_scores(q2, K2)
    i1, t1 = topk_order(s1, k)
    i2, t2 = topk_order(s2, k)
    flat, sc = combine_topk(t1, i1, t2, i2, n_sub, k)
    return {
        "half_idx": np.stack([i1, i2], axis=2),
        "half_score": np.stack([t1, t2], axis=2),
        "idx": flat,
        "score": sc,
        "w": softmax(sc),
    }


def bruteforce_topk(q1, q2, K1, K2, k: int):
    """Exhaustive top-k over all N = n_sub^2 full keys (tiny shapes only).

    Scores every cell (a, b) as <q, [K1[a]; K2[b]]> = s1[a] + s2[b] and sorts all
    N of them under (score descending, flat index ascending).  This is what the
    product-key search must reproduce (overview, how it works: the combination
    gives the right answer among all cells).
    """
    n_sub = K1.shape[1]
    s1 = half_scores(q1, K1)
    s2 = half_scores(q2, K2)
    full = (s1[..., :, None] + s2[..., None, :]).reshape(s1.shape[:-1] + (n_sub * n_sub,))
    return topk_order(full, k)


def forward(inp: dict, cfg, rows_of) -> dict:
    """The whole forward for the tokens in ``inp['x']``.

    ``inp`` holds stored arrays (uint16 bf16 bits or float32): x, W_q, subkeys
    and, with the gate, W1, W2.  ``rows_of(r)`` returns float64 value rows.
    Returns every stage plus ``out`` (float64, before rounding to the output dtype).
    """
    dt = cfg.dtype
    x = to_f64(inp["x"], dt)
    q1, q2 = normalized_query(x, to_f64(inp["W_q"], dt), cfg.H, cfg.d_q, cfg.qk_norm, cfg.norm_eps, dt)
    K1, K2 = normalized_subkeys(to_f64(inp["subkeys"], dt), cfg.qk_norm, cfg.norm_eps, dt)
    res = select(q1, q2, K1, K2, cfg.k)
    res["q1"], res["q2"], res["K1"], res["K2"] = q1, q2, K1, K2
    y = weighted_bag(rows_of, res["idx"], res["w"])
    res["y"] = y
    if cfg.memory_plus:
        res["out"] = memory_plus(y, x, to_f64(inp["W1"], dt), to_f64(inp["W2"], dt), dt)
    else:
        res["out"] = y
    return res


def rows_from_table(table: np.ndarray, dtype: str):
    """``rows_of`` over a materialised table (float32 or bf16 bits)."""
    return lambda r: to_f64(table[np.asarray(r, dtype=np.int64)], dtype)
