"""Pins of the gather-backward oracle (CPU): hand cases, torch autograd of
embedding_bag and softmax as library special cases, and finite differences of the
forward oracle ('Memory Layers at Scale' digest, parallel EmbeddingBag; 'Memory inside
the model' overview, learning without forgetting)."""

import json
import os

import numpy as np
import pytest

from oracle import backward as B
from oracle import pkm as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "backward_hand_cases.json")))


def _rows_of(V):
    V = np.asarray(V, dtype=np.float64)
    return lambda r: V[np.asarray(r, dtype=np.int64)]


def test_hand_case():
    c = GOLD["case"]
    V = np.array(c["V"], float)
    dw = B.grad_weights(_rows_of(V), np.array(c["idx"]), np.array(c["dy"], float), len(V))
    np.testing.assert_array_equal(dw, c["expect_dw"])
    rows, grad = B.grad_rows(np.array(c["idx"]), np.array(c["w"], float), np.array(c["dy"], float), len(V))
    np.testing.assert_array_equal(rows, c["expect_rows"])
    np.testing.assert_array_equal(grad, c["expect_grad"])
    upd = B.sgd_rows(V[rows].astype(np.float32), grad, c["lr"], "f32")
    np.testing.assert_array_equal(upd, c["expect_updated"])


def test_out_of_range_and_duplicates():
    c = GOLD["out_of_range"]
    V = np.array(c["V"], float)
    assert np.array_equal(B.grad_weights(_rows_of(V), np.array(c["idx"]), np.array(c["dy"], float), len(V)),
                          c["expect_dw"])
    rows, _ = B.grad_rows(np.array(c["idx"]), np.array(c["w"], float), np.array(c["dy"], float), len(V))
    assert rows.tolist() == c["expect_rows"]
    d = GOLD["duplicate"]
    rows, grad = B.grad_rows(np.array(d["idx"]), np.array(d["w"], float), np.array(d["dy"], float), 2)
    assert rows.tolist() == d["expect_rows"] and np.array_equal(grad, d["expect_grad"])


def test_softmax_hand_case():
    c = GOLD["softmax"]
    np.testing.assert_allclose(B.softmax_backward(np.array(c["w"]), np.array(c["dw"]), c["group"]), c["expect_ds"],
                               rtol=0, atol=1e-15)


def test_matches_torch_autograd_of_embedding_bag():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    n_rows, dim, n_bags, bag = 40, 12, 30, 7
    V = rng.standard_normal((n_rows, dim))
    idx = rng.integers(0, n_rows, size=(n_bags, bag))
    w = rng.random((n_bags, bag)) + 0.1
    dy = rng.standard_normal((n_bags, dim))
    Vt = torch.tensor(V, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    y = torch.nn.functional.embedding_bag(torch.tensor(idx), Vt, mode="sum", per_sample_weights=wt)
    (y * torch.tensor(dy)).sum().backward()
    np.testing.assert_allclose(B.grad_weights(_rows_of(V), idx, dy, n_rows), wt.grad.numpy(), rtol=1e-13, atol=1e-13)
    rows, grad = B.grad_rows(idx, w, dy, n_rows)
    dense = Vt.grad.numpy()
    touched = np.nonzero(np.any(dense != 0, axis=1))[0]
    np.testing.assert_array_equal(rows, touched)
    np.testing.assert_allclose(grad, dense[rows], rtol=1e-13, atol=1e-13)


def test_softmax_backward_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    s = rng.standard_normal((5, 4 * 8))
    dw = rng.standard_normal((5, 32))
    st = torch.tensor(s, requires_grad=True)
    w = torch.softmax(st.reshape(5, 4, 8), dim=-1).reshape(5, 32)
    (w * torch.tensor(dw)).sum().backward()
    np.testing.assert_allclose(B.softmax_backward(w.detach().numpy(), dw, 8), st.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_finite_differences_of_the_forward_oracle():
    # L = <dy, y>, y from the forward oracle's weighted_bag; L is linear in w and in V,
    # so central differences are exact up to rounding
    rng = np.random.default_rng(2)
    V = rng.standard_normal((10, 6))
    idx = rng.integers(0, 10, size=(3, 4))
    w = rng.random((3, 4))
    dy = rng.standard_normal((3, 6))
    L = lambda ww, VV: float(np.sum(dy * O.weighted_bag(_rows_of(VV), idx, ww)))
    dw = B.grad_weights(_rows_of(V), idx, dy, 10)
    eps = 1e-3
    for b in range(3):
        for j in range(4):
            e = np.zeros_like(w)
            e[b, j] = eps
            np.testing.assert_allclose((L(w + e, V) - L(w - e, V)) / (2 * eps), dw[b, j], rtol=1e-9, atol=1e-10)
    rows, grad = B.grad_rows(idx, w, dy, 10)
    for u, r in enumerate(rows):
        for c in range(6):
            e = np.zeros_like(V)
            e[r, c] = eps
            np.testing.assert_allclose((L(w, V + e) - L(w, V - e)) / (2 * eps), grad[u, c], rtol=1e-9, atol=1e-10)


def _grad_rows_dropping_duplicates(idx, w, dy, n_rows):
    # a plausible slip: a dict assignment instead of accumulation
    acc = {}
    for b in range(idx.shape[0]):
        for j in range(idx.shape[1]):
            acc[int(idx[b, j])] = w[b, j] * dy[b]
    rows = np.array(sorted(acc))
    return rows, np.stack([acc[r] for r in rows])


def test_planted_slip_is_caught():
    d = GOLD["duplicate"]
    _, grad = _grad_rows_dropping_duplicates(np.array(d["idx"]), np.array(d["w"]), np.array(d["dy"], float), 2)
    assert not np.array_equal(grad, d["expect_grad"])
