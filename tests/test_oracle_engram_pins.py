"""Pins of the hashed n-gram lookup oracle (CPU): hand-worked cases, a library special
case, and properties fixed by the mathematics (review of 'Conditional Memory via
Scalable Lookup' (Engram): multi-head hashing, key equations 1 and 2)."""

import json
import math
import os

import numpy as np
import pytest

from oracle import engram as E
from synth import configs as C
from synth import inputs as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "engram_hand_cases.json")))


def _int(v):
    return int(v, 16) if isinstance(v, str) else int(v)


@pytest.mark.parametrize("case", GOLD["hash_cases"], ids=lambda c: str(c["g"]))
def test_hash_hand_cases(case):
    assert E.phi(case["g"], _int(case["m"]), case["P"]) == case["expect"]


@pytest.mark.parametrize("case", GOLD["ngram_cases"], ids=lambda c: f"t{c['t']}n{c['n']}")
def test_ngram_hand_cases(case):
    assert E.ngram(case["ids"], case["seq_len"], case["t"], case["n"], case["vocab"]) == case["expect"]


@pytest.mark.parametrize("case", GOLD["gate_cases"], ids=lambda c: str(len(c["h"][0])))
def test_gate_hand_cases(case):
    a = E.gate(np.array(case["h"], float), np.array(case["e"], float), 0.0)
    np.testing.assert_allclose(a, case["expect_alpha"], rtol=0, atol=1e-15)


def test_forward_hand_case():
    c = GOLD["forward_case"]
    cfg = C.EngramConfig("hand", T=2, seq_len=c["seq_len"], vocab=c["vocab"], zipf_s=1.0, min_order=c["min_order"],
                         n_orders=1, heads=1, head_dim=c["head_dim"], table_rows=c["P"], dtype="f32", norm_eps=0.0)
    rows_of = lambda r: np.stack([np.asarray(r, float), -np.asarray(r, float)], axis=1)
    r = E.forward(cfg, np.array(c["ids"]), np.array(c["h"], np.float32), np.array(c["mult"], np.uint64), rows_of)
    np.testing.assert_array_equal(r["rows"], c["expect_rows"])
    np.testing.assert_allclose(r["alpha"], c["expect_alpha"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r["out64"], c["expect_out"], rtol=0, atol=1e-14)


def test_sigmoid_closed_forms():
    # alpha(h, h) = sigmoid(sqrt(d)) with eps = 0, for any nonzero h
    rng = np.random.default_rng(3)
    for d in (4, 16, 1024):
        h = rng.standard_normal((5, d))
        np.testing.assert_allclose(E.gate(h, h, 0.0), 1 / (1 + math.exp(-math.sqrt(d))), rtol=1e-14)
        np.testing.assert_allclose(E.gate(h, -h, 0.0), 1 / (1 + math.exp(math.sqrt(d))), rtol=1e-12)


def test_gate_scale_invariance():
    rng = np.random.default_rng(4)
    h, e = rng.standard_normal((7, 64)), rng.standard_normal((7, 64))
    np.testing.assert_allclose(E.gate(3.5 * h, 0.01 * e, 0.0), E.gate(h, e, 0.0), rtol=1e-13)


def test_hash_is_a_bijection_of_the_last_token_before_the_modulus():
    # an odd multiplier is invertible modulo 2^64 and XOR with a fixed value is a
    # bijection, so with the prefix fixed, distinct last tokens give distinct h
    m = int(S.engram_multipliers(0, 2, 1, 1)[0, 0])
    hs = set()
    for last in range(5000):
        h = 0
        for tok in (17, last):
            h = ((h ^ tok) * m) % (1 << 64)
        hs.add(h)
    assert len(hs) == 5000
    # and the full hash of the same n-gram under another head's multiplier differs
    m2 = int(S.engram_multipliers(0, 2, 1, 2)[0, 1])
    assert E.phi([17, 3], m, 2097143) != E.phi([17, 3], m2, 2097143)


def test_multipliers_are_odd_and_distinct():
    m = S.engram_multipliers(0, 2, 2, 8)
    assert m.shape == (2, 8) and np.all(m & np.uint64(1) == 1) and len(np.unique(m)) == 16


def test_sequences_are_independent():
    # hashing two sequences together equals hashing each alone (no n-gram crosses a start)
    cfg = C.ENGRAM_CONFIGS["engram_tiny_f32"]
    d = S.make_engram_inputs(cfg, seed=2)
    ids, L = d["ids"], cfg.seq_len
    both = E.hash_rows(ids[:2 * L], L, d["mult"], cfg.table_rows, cfg.min_order, cfg.vocab)
    second = E.hash_rows(ids[L:2 * L], L, d["mult"], cfg.table_rows, cfg.min_order, cfg.vocab)
    np.testing.assert_array_equal(both[L:], second)
    # rows stay inside their own table
    o = np.arange(cfg.n_orders)[None, None, :]
    k = np.arange(cfg.heads)[None, :, None]
    base = (o * cfg.heads + k) * cfg.table_rows
    assert np.all(both >= base) and np.all(both < base + cfg.table_rows)


def test_compress_map():
    cfg = C.ENGRAM_CONFIGS["engram_compress_bf16"]
    d = S.make_engram_inputs(cfg, seed=0, T=300)
    ident = np.arange(cfg.vocab, dtype=np.int32)
    a = E.hash_rows(d["ids"], cfg.seq_len, d["mult"], cfg.table_rows, cfg.min_order, cfg.vocab)
    b = E.hash_rows(d["ids"], cfg.seq_len, d["mult"], cfg.table_rows, cfg.min_order, cfg.vocab, ident)
    np.testing.assert_array_equal(a, b)
    # two tokens mapped to the same concept give the same rows
    cmap = d["compress"]
    t1, t2 = np.nonzero(cmap == cmap[cmap.argmax()])[0][:2]
    ids = np.array([t1, 5, t2, 5], dtype=np.int32)
    r = E.hash_rows(ids, 2, d["mult"], cfg.table_rows, cfg.min_order, cfg.vocab, cmap)
    np.testing.assert_array_equal(r[0], r[2])
    np.testing.assert_array_equal(r[1], r[3])


def test_lookup_is_an_embedding_bag():
    # the library special case: sum-mode EmbeddingBag over (token, head) bags of the orders
    torch = pytest.importorskip("torch")
    cfg = C.ENGRAM_CONFIGS["engram_tiny_f32"]
    d = S.make_engram_inputs(cfg, seed=1)
    rows = E.hash_rows(d["ids"], cfg.seq_len, d["mult"], cfg.table_rows, cfg.min_order, cfg.vocab)
    table = S.engram_table_rows(1, np.arange(cfg.total_rows), cfg.head_dim, "f32").astype(np.float64)
    e = E.lookup(lambda r: table[r], rows, cfg.head_dim)
    bags = torch.from_numpy(rows.reshape(-1, cfg.n_orders))
    ref = torch.nn.functional.embedding_bag(bags, torch.from_numpy(table), mode="sum")
    np.testing.assert_allclose(e, ref.numpy().reshape(cfg.T, cfg.d), rtol=1e-15, atol=1e-17)


def test_residual_and_rounding():
    cfg = C.ENGRAM_CONFIGS["engram_compress_bf16"].with_(T=50)
    d = S.make_engram_inputs(cfg, seed=0, T=50)
    rows_of = lambda r: E.to_f64(S.engram_table_rows(0, r, cfg.head_dim, "bf16"), "bf16")
    a = E.forward(cfg, d["ids"], d["h"], d["mult"], rows_of, d["compress"])
    b = E.forward(cfg.with_(residual=False), d["ids"], d["h"], d["mult"], rows_of, d["compress"])
    np.testing.assert_allclose(a["out64"] - b["out64"], E.to_f64(d["h"], "bf16"), rtol=0, atol=1e-15)
    # one rounding to bf16 of the float64 result
    got = E.to_f64(a["out"], "bf16")
    assert np.all(np.abs(got - a["out64"]) <= np.abs(a["out64"]) * 2.0 ** -8 + 1e-30)


def _phi_reversed(g, m, P):
    return E.phi(list(g)[::-1], m, P)


def _phi_add(g, m, P):
    h = 0
    for tok in g:
        h = ((h + int(tok)) * int(m)) % (1 << 64)
    return h % P


def _phi_no_wrap(g, m, P):
    h = 0
    for tok in g:
        h = (h ^ int(tok)) * int(m)
    return h % P


@pytest.mark.parametrize("slip", [_phi_reversed, _phi_add, _phi_no_wrap])
def test_planted_hash_slips_are_caught(slip):
    wrong = [c for c in GOLD["hash_cases"] if slip(c["g"], _int(c["m"]), c["P"]) != c["expect"]]
    assert wrong, f"{slip.__name__} passes every hand case"
