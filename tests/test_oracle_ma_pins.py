"""Pins of the Memory Attention token-memory oracle (CPU): hand cases, torch's
rms_norm and embedding as library special cases, and per-head properties (summary of
'Memory Attention': how it works, how it differs)."""

import json
import os

import numpy as np
import pytest

from oracle import ma as M
from synth import configs as C
from synth import inputs as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ma_hand_cases.json")))


def test_fold_hand_cases():
    c = GOLD["fold_case"]
    np.testing.assert_allclose(M.fold_table(np.array(c["E"], float), c["n_heads"], None, 0.0), c["expect"],
                               rtol=0, atol=1e-15)
    g = GOLD["gain_case"]
    np.testing.assert_allclose(M.fold_table(np.array(g["E"], float), g["n_heads"], g["gain"], 0.0), g["expect"],
                               rtol=0, atol=1e-15)


def test_values_hand_case():
    c = GOLD["values_case"]
    got = M.values(np.array(c["Ebar"], np.float32), c["ids"], np.array(c["K"], np.float32), "f32")
    np.testing.assert_array_equal(got, c["expect"])


def test_fold_matches_torch_rms_norm_per_head():
    torch = pytest.importorskip("torch")
    cfg = C.MA_CONFIGS["ma_tiny_f32"]
    d = S.make_ma_inputs(cfg, seed=3)
    E = d["E"].astype(np.float64)
    ours = M.fold_table(E, cfg.n_heads, d["gain"], cfg.norm_eps)
    x = torch.from_numpy(E).view(cfg.vocab, cfg.n_heads, cfg.head_dim)
    g = torch.from_numpy(d["gain"].astype(np.float64)).view(cfg.n_heads, cfg.head_dim)
    ref = torch.stack([torch.nn.functional.rms_norm(x[:, h], (cfg.head_dim,), weight=g[h], eps=cfg.norm_eps)
                       for h in range(cfg.n_heads)], dim=1).reshape(cfg.vocab, cfg.d_v)
    np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-13, atol=1e-15)


def test_fold_unit_rms_per_head_and_scale_invariance():
    rng = np.random.default_rng(0)
    E = rng.standard_normal((50, 64))
    f = M.fold_table(E, 4, None, 0.0).reshape(50, 4, 16)
    np.testing.assert_allclose(np.sqrt(np.mean(f * f, axis=-1)), 1.0, rtol=1e-14)
    # each head slice is scale-invariant on its own
    E2 = E.copy()
    E2[:, 16:32] *= 7.0
    np.testing.assert_allclose(M.fold_table(E2, 4, None, 0.0), M.fold_table(E, 4, None, 0.0), rtol=1e-14)


def test_values_match_torch_embedding():
    torch = pytest.importorskip("torch")
    cfg = C.MA_CONFIGS["ma_tiny_f32"]
    d = S.make_ma_inputs(cfg, seed=1)
    Eb = M.store(M.fold_table(d["E"].astype(np.float64), cfg.n_heads, d["gain"], cfg.norm_eps), "f32")
    got = M.values(Eb, d["ids"], d["K"], "f32")
    ref = torch.nn.functional.embedding(torch.from_numpy(d["ids"].astype(np.int64)),
                                        torch.from_numpy(Eb.astype(np.float64))) + torch.from_numpy(d["K"].astype(np.float64))
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=0)


def _fold_whole_row(E, n_heads, gain, eps):
    return M.fold_table(E, 1, gain, eps)


def test_planted_slip_norm_over_whole_row_is_caught():
    c = GOLD["fold_case"]
    got = _fold_whole_row(np.array(c["E"], float), c["n_heads"], None, 0.0)
    assert not np.allclose(got, c["expect"], atol=1e-6)
