"""Oracle of the Memory Attention token-memory values (TEST INFRASTRUCTURE; float64 NumPy).

Source: the summary of "Memory Attention" (replacing the attention value projection
with a per-layer token memory), cited by section:

* "how it works": every layer keeps a trainable table E of vocabulary size by d_v;
  the input token id s reads E[s], an RMSNorm is applied to each token vector within
  every key/value head, giving M, and the values are V = K + M (no value projection).
* "how it differs": at inference the norm can be folded into the table beforehand,
  E_bar[i] = Norm(E[i]), so that building the values online is one lookup and one
  elementwise add, V = K + E_bar[s].

Readings (listed with their reasons in the design notes of the repository):

* the norm is RMSNorm v / sqrt(mean(v^2) + eps) over each head's head_dim slice,
  times an optional per-channel gain (the page counts extra norm parameters);
* the folded table is stored in the table's type (rounded once from float64); the
  values are K + E_bar[s] rounded once to the storage type;
* a token id outside [0, vocab) reads no memory: V = K.
"""

from __future__ import annotations

import numpy as np

from .pkm import f64_to_bf16_bits, to_f64


def fold_table(E64: np.ndarray, n_heads: int, gain, eps: float) -> np.ndarray:
    """E_bar = RMSNorm per head slice of every row, times the gain (float64)."""
    V, d_v = E64.shape
    hd = d_v // n_heads
    x = E64.reshape(V, n_heads, hd)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = y.reshape(V, d_v)
    if gain is not None:
        y = y * np.asarray(gain, dtype=np.float64)[None, :]
    return y


def store(v64: np.ndarray, dtype: str) -> np.ndarray:
    return v64.astype(np.float32) if dtype == "f32" else f64_to_bf16_bits(v64)


def values(Ebar_stored: np.ndarray, ids, K_stored: np.ndarray, dtype: str) -> np.ndarray:
    """V = K + E_bar[s] (float64 of the stored operands); out-of-range ids add nothing."""
    Eb = to_f64(Ebar_stored, dtype)
    K = to_f64(K_stored, dtype)
    ids = np.asarray(ids, dtype=np.int64)
    ok = (ids >= 0) & (ids < Eb.shape[0])
    out = K.copy()
    out[ok] += Eb[ids[ok]]
    return out
