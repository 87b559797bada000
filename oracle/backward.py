"""Oracle of the gather backward and the sparse update (TEST INFRASTRUCTURE; float64 NumPy).

Sources, cited by page title and section:

* "Memory Layers at Scale" digest, parallel EmbeddingBag: the value read is a weighted
  EmbeddingBag in the forward pass, y[b] = sum over j of w[b, j] * V[idx[b, j]]; its
  backward follows from that sum by the chain rule: with dy = dL/dy,
    dL/dw[b, j] = <dy[b], V[idx[b, j]]>,
    dL/dV[r]    = sum over (b, j) with idx[b, j] = r of w[b, j] * dy[b]   (zero elsewhere).
* "Memory inside the model" overview, learning without forgetting: a fact lives in a
  few slots, so training can edit only the touched slots; the update here is plain
  SGD on the rows that received a gradient, V[r] <- V[r] - lr * dL/dV[r].
* The weights are a softmax of the scores per head (digest, core idea), so
  dL/ds[j] = w[j] * (dL/dw[j] - sum over j' of w[j'] * dL/dw[j']) within each group.

Readings (listed with their reasons in the design notes of the repository): an index
outside [0, n_rows) read nothing in the forward and receives no gradient; the distinct
rows are reported in ascending order; the update rounds V[r] - lr * grad once to the
table's storage type.
"""

from __future__ import annotations

import numpy as np

from .pkm import f64_to_bf16_bits, to_f64


def grad_weights(rows_of, idx: np.ndarray, dy: np.ndarray, n_rows: int) -> np.ndarray:
    """dL/dw[b, j] = <dy[b], V[idx[b, j]]> (0 for an out-of-range index); float64 [n_bags, bag].

    ``rows_of(r)`` returns the float64 rows r of the table."""
    idx = np.asarray(idx, dtype=np.int64)
    dy = np.asarray(dy, dtype=np.float64)
    ok = (idx >= 0) & (idx < n_rows)
    rows = rows_of(np.where(ok, idx, 0).reshape(-1)).reshape(idx.shape + (dy.shape[1],))
    return np.where(ok, np.einsum("bjc,bc->bj", rows, dy), 0.0)


def grad_rows(idx: np.ndarray, w: np.ndarray, dy: np.ndarray, n_rows: int):
    """Distinct rows touched (ascending) and dL/dV of each: (rows [U] int64, grad [U, dim] float64)."""
    idx = np.asarray(idx, dtype=np.int64)
    w = np.asarray(w, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    acc = {}
    for b in range(idx.shape[0]):
        for j in range(idx.shape[1]):
            r = int(idx[b, j])
            if 0 <= r < n_rows:
                acc[r] = acc.get(r, 0.0) + w[b, j] * dy[b]
    rows = np.array(sorted(acc), dtype=np.int64)
    grad = np.stack([acc[r] for r in rows]) if len(rows) else np.zeros((0, dy.shape[1]))
    return rows, grad


def softmax_backward(w: np.ndarray, dw: np.ndarray, group: int) -> np.ndarray:
    """dL/ds for w = softmax(s) over consecutive groups of `group` entries of each bag."""
    w = np.asarray(w, dtype=np.float64)
    dw = np.asarray(dw, dtype=np.float64)
    n_bags, bag = w.shape
    wg = w.reshape(n_bags, bag // group, group)
    dg = dw.reshape(n_bags, bag // group, group)
    return (wg * (dg - np.sum(wg * dg, axis=-1, keepdims=True))).reshape(n_bags, bag)


def sgd_rows(old_stored: np.ndarray, grad: np.ndarray, lr: float, dtype: str) -> np.ndarray:
    """Updated stored rows: V[r] - lr * grad, rounded once to the storage type."""
    v = to_f64(old_stored, dtype) - lr * np.asarray(grad, dtype=np.float64)
    return v.astype(np.float32) if dtype == "f32" else f64_to_bf16_bits(v)
