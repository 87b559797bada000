"""Oracle of the hashed n-gram lookup (TEST INFRASTRUCTURE; float64 NumPy).

Source: the review of "Conditional Memory via Scalable Lookup" (Engram), cited by
section and equation:

* section "sparse retrieval", item "multi-head hashing": the n-grams ending at a
  token (2-grams, 3-grams, ...) are each hashed by several independent hash
  functions into the indices of large embedding tables; key equation 1,
  e_{t,n,k} = E_{n,k}[phi_{n,k}(g_{t,n})].
* same section, item "tokenizer compression": token ids that mean the same thing
  are first mapped onto one id.
* section "context-aware fusion", item "context-aware gating" and key equation 2:
  alpha_t = sigmoid(RMSNorm(h_t) . RMSNorm(e_t) / sqrt(d)), from the current hidden
  state h_t and the retrieved embedding e_t; item "residual connection": the result
  is added to h_t.

Readings of points the page leaves open (listed with their reasons in the design
notes of the repository):

* phi_{n,k} is a multiplicative-XOR fold: starting from 0, for each token j of the
  n-gram, oldest first, h <- ((h XOR id_j) * m_{n,k}) mod 2^64; then
  phi = h mod P, with one odd 64-bit multiplier m_{n,k} per (order, head), passed
  in as an input, and P the number of rows of every table.
* an n-gram that reaches back past the start of its sequence uses id 0 for the
  missing tokens; an id outside [0, vocab) is read as 0 too.
* e_t is the concatenation over heads k of the sum over orders n of e_{t,n,k}
  (so heads * head_dim = d matches h_t with no projection); the tables E_{n,k}
  are stacked into one table whose row ((n - n_min) * heads + k) * P + phi holds
  E_{n,k}[phi].
* RMSNorm v / sqrt(mean(v^2) + eps), unit gain; output alpha_t * e_t, or
  h_t + alpha_t * e_t with the residual; the depthwise convolution the page lists
  after the gate is left out (its width and activation are not given).
* arithmetic in float64 on the stored values; the output is rounded once to the
  storage type.
"""

from __future__ import annotations

import numpy as np

from .pkm import f64_to_bf16_bits, to_f64

M64 = 1 << 64


def normalize_id(tok: int, vocab: int, compress=None) -> int:
    """The id the hash sees: out-of-range ids read as 0, then the optional vocabulary
    map (sparse retrieval, tokenizer compression)."""
    tok = int(tok)
    if tok < 0 or tok >= vocab:
        tok = 0
    return int(compress[tok]) if compress is not None else tok


def ngram(ids, seq_len: int, t: int, n: int, vocab: int, compress=None) -> list[int]:
    """g_{t,n}: the n ids ending at position t, oldest first; positions before the
    start of t's sequence contribute id 0."""
    start = (t // seq_len) * seq_len
    return [normalize_id(ids[j], vocab, compress) if j >= start else 0 for j in range(t - n + 1, t + 1)]


def phi(g, m: int, P: int) -> int:
    """phi_{n,k}(g): multiplicative-XOR fold of the n-gram modulo 2^64, then mod P
    (multi-head hashing)."""
    h = 0
    for tok in g:
        h = ((h ^ int(tok)) * int(m)) % M64
    return h % P


def hash_rows(ids, seq_len: int, mult, P: int, min_order: int, vocab: int, compress=None) -> np.ndarray:
    """Row of the stacked table read for every (token, head, order): [T, heads, n_orders]
    int64, row = (o * heads + k) * P + phi_{n,k}(g_{t,n}) with n = min_order + o
    (key equation 1)."""
    mult = np.asarray(mult, dtype=np.uint64)
    n_orders, heads = mult.shape
    T = len(ids)
    rows = np.empty((T, heads, n_orders), dtype=np.int64)
    for t in range(T):
        for o in range(n_orders):
            g = ngram(ids, seq_len, t, min_order + o, vocab, compress)
            for k in range(heads):
                rows[t, k, o] = (o * heads + k) * P + phi(g, int(mult[o, k]), P)
    return rows


def lookup(rows_of, rows: np.ndarray, head_dim: int) -> np.ndarray:
    """e_t = concat over heads k of sum over orders of E_{n,k}[phi] (float64, [T, heads * head_dim]).

    ``rows_of(r)`` returns the float64 rows r of the stacked table."""
    T, heads, n_orders = rows.shape
    e = np.zeros((T, heads, head_dim), dtype=np.float64)
    for o in range(n_orders):
        e += rows_of(rows[:, :, o].reshape(-1)).reshape(T, heads, head_dim)
    return e.reshape(T, heads * head_dim)


def rmsnorm(v: np.ndarray, eps: float) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)


def gate(h: np.ndarray, e: np.ndarray, eps: float) -> np.ndarray:
    """alpha_t = sigmoid(RMSNorm(h_t) . RMSNorm(e_t) / sqrt(d)) (key equation 2), [T]."""
    d = h.shape[-1]
    z = np.sum(rmsnorm(h, eps) * rmsnorm(e, eps), axis=-1) / np.sqrt(d)
    return 1.0 / (1.0 + np.exp(-z))


def forward(cfg, ids, h_stored, mult, rows_of, compress=None):
    """The whole lookup: rows, e (float64), alpha (float64) and the output as stored
    values (float32, or bf16 bits).  ``h_stored`` holds the stored hidden states."""
    rows = hash_rows(ids, cfg.seq_len, mult, cfg.table_rows, cfg.min_order, cfg.vocab, compress)
    e = lookup(rows_of, rows, cfg.head_dim)
    h = to_f64(h_stored, cfg.dtype)
    alpha = gate(h, e, cfg.norm_eps)
    out = alpha[:, None] * e
    if cfg.residual:
        out = out + h
    stored = out.astype(np.float32) if cfg.dtype == "f32" else f64_to_bf16_bits(out)
    return {"rows": rows, "e": e, "alpha": alpha, "out64": out, "out": stored}
