"""Pins of the oracle to things other than itself (CPU only).

Each test checks the oracle against a hand-worked case, a closed form, an
invariant, a different library routine, or brute force on tiny inputs, chosen
so that a plausible slip in the oracle (a dropped half, a swapped flat index, a
reversed tie-break, a missing max-subtraction) fails at least one of them.
The mutation tests at the end plant such slips in a copy of the oracle and
check that the pins catch them.
"""

import heapq
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import pkm as O
from synth import CONFIGS
from synth import inputs as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def _case_select(c):
    x = np.array(c["x"], dtype=np.float64)
    q1, q2 = O.normalized_query(x, np.array(c["W_q"], float), c["H"], c["d_q"], False, 1e-6, "f32")
    K1, K2 = O.normalized_subkeys(np.array(c["subkeys"], float), False, 1e-6, "f32")
    return O.select(q1, q2, K1, K2, c["k"]), (q1, q2, K1, K2)


def test_hand_product_key_case():
    c = GOLD["product_key_case"]
    r, (q1, q2, K1, K2) = _case_select(c)
    assert r["half_idx"][0, 0].tolist() == c["expect_half_idx"]
    np.testing.assert_allclose(r["half_score"][0, 0], c["expect_half_score"], rtol=0, atol=1e-15)
    assert r["idx"][0, 0].tolist() == c["expect_idx"]
    np.testing.assert_allclose(r["score"][0, 0], c["expect_score"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r["w"][0, 0], c["expect_w"], rtol=1e-15)
    V = np.array(c["values"], dtype=np.float64)
    y = O.weighted_bag(lambda rr: V[rr], r["idx"], r["w"])
    np.testing.assert_allclose(y[0], c["expect_y"], rtol=1e-15)
    bi, bs = O.bruteforce_topk(q1, q2, K1, K2, c["k"])
    assert bi[0, 0].tolist() == c["expect_idx"]


def test_hand_tie_case_lowest_index_wins():
    c = GOLD["tie_case"]
    r, _ = _case_select(c)
    assert r["idx"][0, 0].tolist() == c["expect_idx"]
    np.testing.assert_allclose(r["w"][0, 0], c["expect_w"], rtol=1e-15)


def test_hand_rmsnorm():
    c = GOLD["rmsnorm_case"]
    np.testing.assert_allclose(O.rmsnorm(np.array(c["v"], float), 0.0), c["expect"], rtol=1e-14)


def test_hand_rmsnorm_eps_inside_the_root():
    c = GOLD["rmsnorm_eps_case"]
    np.testing.assert_allclose(O.rmsnorm(np.array(c["v"], float), c["eps"]), c["expect"], rtol=1e-14)
    # the worked closed form: v / sqrt(mean(v^2) + eps) = [3, 4] / sqrt(13)
    np.testing.assert_allclose(c["expect"], np.array([3.0, 4.0]) / math.sqrt(13.0), rtol=1e-15)


class _Cfg:
    """The fields of a workload that the oracle's forward reads."""

    def __init__(self, **kw):
        self.__dict__.update(dict(dtype="f32", qk_norm=False, norm_eps=1e-6, memory_plus=False), **kw)


def _two_head_forward():
    c = GOLD["two_head_forward_case"]
    cfg = _Cfg(H=c["H"], d_q=c["d_q"], k=c["k"])
    inp = {"x": np.array(c["x"], np.float32), "W_q": np.array(c["W_q"], np.float32),
           "subkeys": np.array(c["subkeys"], np.float32)}
    V = np.array(c["values"], dtype=np.float64)
    return c, O.forward(inp, cfg, lambda r: V[np.asarray(r)])


def test_hand_two_head_forward():
    """Two heads through the whole forward: each head's own W_q columns and sub-key lists,
    per-head softmax, and one bag over both heads' rows (a row picked twice counts twice)."""
    c, r = _two_head_forward()
    assert r["half_idx"][0].tolist() == c["expect_half_idx"]
    np.testing.assert_allclose(r["half_score"][0], c["expect_half_score"], rtol=0, atol=1e-15)
    assert r["idx"][0].tolist() == c["expect_idx"]
    np.testing.assert_allclose(r["score"][0], c["expect_score"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r["w"][0], c["expect_w"], rtol=1e-15)
    np.testing.assert_allclose(r["out"][0], c["expect_y"], rtol=1e-15)
    # the stored weights are the logistic of each head's score gap (closed form)
    for h, gap in enumerate(c["expect_gap"]):
        np.testing.assert_allclose(c["expect_w"][h], [1 / (1 + math.exp(-gap)), 1 / (1 + math.exp(gap))], rtol=1e-15)
    s = lambda z: 1 / (1 + math.exp(-z))
    np.testing.assert_allclose(c["expect_y"], [s(0.5) + s(1.5), s(-0.5) + 2 * s(-1.5)], rtol=1e-15)


def _projections_equal_when_stored(d, seed):
    """x [1, 2] and two weight matrices whose exact products x W differ (by 2^-11, alternating in
    sign) but round to the same bf16 values a (bf16-exact, in [1, 2), where half an ulp is 2^-8)."""
    rng = np.random.default_rng(seed)
    a = O.bf16_bits_to_f64(O.f64_to_bf16_bits(rng.uniform(1.0, 2.0, d)))
    s = np.where(np.arange(d) % 2 == 0, 1.0, -1.0) * 2.0 ** -12
    x = np.array([[1.0, 1.0]])
    Wa, Wb = np.stack([a, s]), np.stack([a, -s])
    assert not np.array_equal(x @ Wa, x @ Wb)
    assert np.array_equal(O.f64_to_bf16_bits(x @ Wa), O.f64_to_bf16_bits(a[None]))
    assert np.array_equal(O.f64_to_bf16_bits(x @ Wb), O.f64_to_bf16_bits(a[None]))
    return x, Wa, Wb


def test_bf16_query_is_normalised_from_its_stored_projection():
    """bf16 workloads store q = x W_q in bf16 before the qk-norm reads it (the type a bf16
    product returns): two projections that store the same bf16 values give the same q-hat,
    bit for bit.  The case is one where normalising the exact products would not (so a
    missing or misplaced rounding fails here)."""
    d = 64
    x, Wa, Wb = _projections_equal_when_stored(d, seed=10)
    qa = np.concatenate(O.normalized_query(x, Wa, 1, d, True, 0.0, "bf16"), axis=-1)
    qb = np.concatenate(O.normalized_query(x, Wb, 1, d, True, 0.0, "bf16"), axis=-1)
    np.testing.assert_array_equal(qa, qb)
    ea, eb = (O.round_stored(O.rmsnorm(x @ W, 0.0), "bf16") for W in (Wa, Wb))
    assert (ea != eb).sum() >= 3
    # fp32 workloads keep the exact product
    fa = np.concatenate(O.normalized_query(x, Wa, 1, d, True, 0.0, "f32"), axis=-1)
    fb = np.concatenate(O.normalized_query(x, Wb, 1, d, True, 0.0, "f32"), axis=-1)
    assert not np.array_equal(fa, fb)


def test_bf16_gate_reads_its_stored_projection():
    """The same for z = x W1 of the Memory+ gate: equal stored z, equal output; the exact
    products would give different gated rows."""
    d = 64
    x, Wa, Wb = _projections_equal_when_stored(d, seed=10)
    y = np.ones((1, d))
    oa = O.memory_plus(y, x, Wa, np.eye(d), "bf16")
    ob = O.memory_plus(y, x, Wb, np.eye(d), "bf16")
    np.testing.assert_array_equal(oa, ob)
    ga, gb = (O.round_stored(y * O.silu(x @ W), "bf16") for W in (Wa, Wb))
    assert (ga != gb).sum() >= 3


def test_hand_memory_plus():
    c = GOLD["memory_plus_case"]
    out = O.memory_plus(np.array(c["y"], float), np.array(c["x"], float), np.array(c["W1"], float),
                        np.array(c["W2"], float), "f32")
    np.testing.assert_allclose(out, c["expect"], rtol=1e-15, atol=1e-300)


def test_memory_plus_identity_closed_form():
    rng = np.random.default_rng(3)
    y, x = rng.standard_normal((5, 7)), rng.standard_normal((5, 7))
    out = O.memory_plus(y, x, np.eye(7), np.eye(7), "f32")
    np.testing.assert_allclose(out, y * x / (1 + np.exp(-x)), rtol=1e-14)


# ---------------------------------------------------------------------------------
# product-key search == exhaustive search over all N cells


def _rand_problem(rng, T, H, d_h, n, ties=None):
    q1 = rng.standard_normal((T, H, d_h))
    q2 = rng.standard_normal((T, H, d_h))
    K1 = rng.standard_normal((H, n, d_h))
    K2 = rng.standard_normal((H, n, d_h))
    if ties == "dup_keys":          # duplicated sub-keys: equal half scores
        m = len(range(1, n, 2))
        K1[:, 1::2] = K1[:, 0::2][:, :m]
        K2[:, n // 2:] = K2[:, : n - n // 2]
    elif ties == "zero_query":      # every score zero: pure index order
        q1[:] = 0.0
        q2[:] = 0.0
    elif ties == "integer":         # small integers: many exact ties, exact sums
        q1 = rng.integers(-2, 3, (T, H, d_h)).astype(float)
        q2 = rng.integers(-2, 3, (T, H, d_h)).astype(float)
        K1 = rng.integers(-1, 2, (H, n, d_h)).astype(float)
        K2 = rng.integers(-1, 2, (H, n, d_h)).astype(float)
    elif ties == "neg_zero":        # -0.0 and +0.0 scores must tie
        q1 = rng.integers(-1, 2, (T, H, d_h)).astype(float)
        q2 = -np.zeros((T, H, d_h))
        K1 = rng.integers(-1, 2, (H, n, d_h)).astype(float)
        K2 = rng.integers(-1, 2, (H, n, d_h)).astype(float)
    return q1, q2, K1, K2


@pytest.mark.parametrize("n,k", [(8, 1), (8, 4), (8, 8), (16, 5), (16, 16), (13, 7)])
@pytest.mark.parametrize("ties", [None, "dup_keys", "zero_query", "integer", "neg_zero"])
def test_product_key_equals_bruteforce_tiny(n, k, ties):
    """Figure D of the overview: 8 + 8 comparisons find the best of 64 cells."""
    for seed in range(8):
        rng = np.random.default_rng([n, k, seed])
        q1, q2, K1, K2 = _rand_problem(rng, T=6, H=2, d_h=3, n=n, ties=ties)
        r = O.select(q1, q2, K1, K2, k)
        bi, bs = O.bruteforce_topk(q1, q2, K1, K2, k)
        np.testing.assert_array_equal(r["idx"], bi)
        np.testing.assert_array_equal(r["score"], bs)


def test_product_key_equals_bruteforce_tiny_fp32_workload():
    """Product keys vs all 65,536 cells on the small fp32 workload (first 48 tokens)."""
    cfg = CONFIGS["tiny_fp32_65k"]
    inp = S.make_inputs(cfg, seed=0, T=48)
    q1, q2 = O.normalized_query(inp["x"].astype(float), inp["W_q"].astype(float), cfg.H, cfg.d_q,
                                cfg.qk_norm, cfg.norm_eps, cfg.dtype)
    K1, K2 = O.normalized_subkeys(inp["subkeys"].astype(float), cfg.qk_norm, cfg.norm_eps, cfg.dtype)
    r = O.select(q1, q2, K1, K2, cfg.k)
    bi, bs = O.bruteforce_topk(q1, q2, K1, K2, cfg.k)
    np.testing.assert_array_equal(r["idx"], bi)
    np.testing.assert_array_equal(r["score"], bs)


def test_product_key_equals_bruteforce_bf16_qknorm():
    """Same pin with qk-norm and bf16 rounding of the normalised query and keys."""
    cfg = CONFIGS["pkm_1m_bf16"].with_(n_sub=64, d_q=64, H=2, T=16, d_model=96)
    inp = S.make_inputs(cfg, seed=5)
    q1, q2 = O.normalized_query(O.to_f64(inp["x"], "bf16"), O.to_f64(inp["W_q"], "bf16"), cfg.H, cfg.d_q,
                                True, cfg.norm_eps, "bf16")
    K1, K2 = O.normalized_subkeys(O.to_f64(inp["subkeys"], "bf16"), True, cfg.norm_eps, "bf16")
    r = O.select(q1, q2, K1, K2, cfg.k)
    bi, _ = O.bruteforce_topk(q1, q2, K1, K2, cfg.k)
    np.testing.assert_array_equal(r["idx"], bi)


def _python_topk(vals, k):
    """Repeated extraction of the best remaining element (score desc, index asc)."""
    remaining = list(range(len(vals)))
    out = []
    for _ in range(k):
        best = remaining[0]
        for i in remaining[1:]:
            if vals[i] > vals[best] or (vals[i] == vals[best] and i < best):
                best = i
        out.append(best)
        remaining.remove(best)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_topk_order_matches_python_selection(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(5, 40))
    k = int(rng.integers(1, n + 1))
    vals = rng.integers(-3, 4, n).astype(float) * 0.5
    vals[rng.integers(0, n)] = -0.0
    idx, sc = O.topk_order(vals[None, :], k)
    assert idx[0].tolist() == _python_topk(list(vals), k)
    # a second library: heapq.nlargest on (score, -index) keys
    assert idx[0].tolist() == [-i for _, i in heapq.nlargest(k, [(v, -i) for i, v in enumerate(vals)])]


# ---------------------------------------------------------------------------------
# softmax, gather, norm, heads


def test_softmax_invariants_and_two_point_closed_form():
    rng = np.random.default_rng(1)
    s = -np.sort(-rng.standard_normal((50, 32)), axis=1)
    w = O.softmax(s)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert (w > 0).all()
    assert (np.diff(w, axis=1) <= 0).all()
    a, b = 1.7, -0.4
    np.testing.assert_allclose(O.softmax(np.array([a, b])), [1 / (1 + math.exp(b - a)), 1 / (1 + math.exp(a - b))],
                               rtol=1e-15)
    # large scores: no overflow thanks to max-subtraction
    np.testing.assert_allclose(O.softmax(np.array([1000.0, 1000.0])), [0.5, 0.5])


def test_weighted_bag_matches_torch_embedding_bag():
    rng = np.random.default_rng(2)
    V = rng.standard_normal((50, 12))
    idx = rng.integers(0, 50, (7, 3, 4))
    idx[0, 0, 1] = idx[0, 1, 2]  # a row chosen twice counts twice
    w = rng.random((7, 3, 4))
    y = O.weighted_bag(lambda r: V[r], idx, w)
    ref = torch.nn.functional.embedding_bag(torch.from_numpy(idx.reshape(7, -1)), torch.from_numpy(V),
                                            mode="sum", per_sample_weights=torch.from_numpy(w.reshape(7, -1)))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-14)


def test_weighted_bag_one_hot_and_linearity():
    rng = np.random.default_rng(4)
    V = rng.standard_normal((30, 8))
    idx = rng.integers(0, 30, (5, 1, 6))
    w = np.zeros((5, 1, 6))
    w[:, 0, 2] = 1.0
    np.testing.assert_array_equal(O.weighted_bag(lambda r: V[r], idx, w), V[idx[:, 0, 2]])
    w = rng.random((5, 1, 6))
    np.testing.assert_allclose(O.weighted_bag(lambda r: 3.0 * V[r], idx, w),
                               3.0 * O.weighted_bag(lambda r: V[r], idx, w), rtol=1e-14)


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((9, 64))
    r = O.rmsnorm(v, 0.0)
    np.testing.assert_allclose(np.sqrt((r * r).mean(axis=1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(O.rmsnorm(7.5 * v, 0.0), r, rtol=1e-14)


def test_selection_invariant_to_query_scale_with_qknorm():
    """qk-norm makes the selection independent of the scale of W_q (power of two: bf16-exact)."""
    cfg = CONFIGS["pkm_1m_bf16"].with_(n_sub=32, d_q=32, H=2, T=8, d_model=48, k=8)
    inp = S.make_inputs(cfg, seed=9)
    x = O.to_f64(inp["x"], "bf16")
    Wq = O.to_f64(inp["W_q"], "bf16")
    K1, K2 = O.normalized_subkeys(O.to_f64(inp["subkeys"], "bf16"), True, 0.0, "bf16")
    a = O.select(*O.normalized_query(x, Wq, 2, 32, True, 0.0, "bf16"), K1, K2, 8)
    b = O.select(*O.normalized_query(x, 4.0 * Wq, 2, 32, True, 0.0, "bf16"), K1, K2, 8)
    np.testing.assert_array_equal(a["idx"], b["idx"])


def test_heads_sum_decomposition():
    """y with H heads equals the sum of the y's of each head alone (one bag of H*k rows)."""
    rng = np.random.default_rng(6)
    H, T, d_h, n, k = 3, 5, 4, 9, 4
    q1, q2, K1, K2 = _rand_problem(rng, T, H, d_h, n)
    V = rng.standard_normal((n * n, 6))
    r = O.select(q1, q2, K1, K2, k)
    y = O.weighted_bag(lambda rr: V[rr], r["idx"], r["w"])
    acc = np.zeros_like(y)
    for h in range(H):
        rh = O.select(q1[:, h:h + 1], q2[:, h:h + 1], K1[h:h + 1], K2[h:h + 1], k)
        acc += O.weighted_bag(lambda rr: V[rr], rh["idx"], rh["w"])
    np.testing.assert_allclose(y, acc, rtol=1e-13)


def test_token_permutation_equivariance():
    rng = np.random.default_rng(7)
    q1, q2, K1, K2 = _rand_problem(rng, 9, 2, 5, 11)
    perm = rng.permutation(9)
    a = O.select(q1, q2, K1, K2, 6)
    b = O.select(q1[perm], q2[perm], K1, K2, 6)
    np.testing.assert_array_equal(a["idx"][perm], b["idx"])


# ---------------------------------------------------------------------------------
# rounding helpers


def test_f64_to_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(8)
    v = (rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.f64_to_bf16_bits(v.astype(np.float64)), ref)


def test_f64_to_bf16_single_rounding_halfway():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to even (1.0)
    assert O.f64_to_bf16_bits(np.array([1 + 2 ** -8]))[0] == 0x3F80
    # just above halfway rounds up, even where a float32 step would have rounded to the tie
    assert O.f64_to_bf16_bits(np.array([1 + 2 ** -8 + 2 ** -40]))[0] == 0x3F81
    assert O.f64_to_bf16_bits(np.array([1 + 3 * 2 ** -8]))[0] == 0x3F82
    assert O.f64_to_bf16_bits(np.array([-2.0]))[0] == 0xC000


# ---------------------------------------------------------------------------------
# planted slips: copies of oracle steps with a deliberate mistake must fail the pins


def _select_with(combine_fn, topk_fn, q1, q2, K1, K2, k):
    n_sub = K1.shape[1]
    s1, s2 = O.half_scores(q1, K1), O.half_scores(q2, K2)
    i1, t1 = topk_fn(s1, k)
    i2, t2 = topk_fn(s2, k)
    return combine_fn(t1, i1, t2, i2, n_sub, k)


def _combine_swapped_flat(s1, i1, s2, i2, n_sub, k):
    return O.combine_topk(s2, i2, s1, i1, n_sub, k)  # flat = b * n + a


def _topk_reversed_ties(scores, k):
    n = scores.shape[-1]
    ar = np.broadcast_to(-np.arange(n), scores.shape)
    order = np.lexsort((ar, -scores), axis=-1)[..., :k]
    return order, np.take_along_axis(scores, order, axis=-1)


def _combine_first_half_only(s1, i1, s2, i2, n_sub, k):
    return O.combine_topk(s1, i1, 0.0 * s2, i2, n_sub, k)


@pytest.mark.parametrize("slip", ["swapped_flat", "reversed_ties", "dropped_half"])
def test_pins_catch_planted_slips(slip):
    combine = {"swapped_flat": _combine_swapped_flat, "dropped_half": _combine_first_half_only}.get(slip, O.combine_topk)
    topk = _topk_reversed_ties if slip == "reversed_ties" else O.topk_order
    caught = False
    for ties in [None, "integer"]:
        for seed in range(4):
            rng = np.random.default_rng([seed, 99])
            q1, q2, K1, K2 = _rand_problem(rng, T=6, H=1, d_h=3, n=8, ties=ties)
            got, _ = _select_with(combine, topk, q1, q2, K1, K2, 4)
            want, _ = O.bruteforce_topk(q1, q2, K1, K2, 4)
            caught |= not np.array_equal(got, want)
    assert caught, f"planted slip {slip} was not caught by the brute-force pin"


def _project_query_interleaved(x, W_q, H, d_q):
    """Slip: head h taken as every H-th column from h (a reshape in the wrong order)."""
    q = x @ W_q
    return q.reshape(x.shape[0], d_q, H).transpose(0, 2, 1)


def _rmsnorm_eps_outside(v, eps):
    """Slip: eps added after the square root."""
    return v / (np.sqrt(np.mean(v * v, axis=-1, keepdims=True)) + eps)


def _normalized_query_from_exact_product(x, W_q, H, d_q, qk_norm, eps, dtype):
    """Slip: the norm reads the exact product instead of the stored q."""
    q = O.project_query(x, W_q, H, d_q)
    q = O.rmsnorm(q, eps) if qk_norm else q
    return O.split_halves(O.round_stored(q, dtype))


def _memory_plus_from_exact_product(y, x, W1, W2, dtype):
    """Slip: the gate reads the exact x W1 instead of the stored z."""
    return O.round_stored(y * O.silu(x @ W1), dtype) @ W2


@pytest.mark.parametrize("slip,target,pin", [
    ("head_split_transposed", "project_query", test_hand_two_head_forward),
    ("eps_outside_the_root", "rmsnorm", test_hand_rmsnorm_eps_inside_the_root),
    ("query_norm_of_the_exact_product", "normalized_query", test_bf16_query_is_normalised_from_its_stored_projection),
    ("gate_of_the_exact_product", "memory_plus", test_bf16_gate_reads_its_stored_projection),
])
def test_pins_catch_planted_oracle_slips(monkeypatch, slip, target, pin):
    """A wrong head split, eps outside the square root, or a norm or gate that reads the exact
    product instead of the stored one, planted in the oracle's own step, fails the pin of
    that step."""
    pin()   # the true oracle passes
    monkeypatch.setattr(O, target, {"project_query": _project_query_interleaved,
                                    "rmsnorm": _rmsnorm_eps_outside,
                                    "normalized_query": _normalized_query_from_exact_product,
                                    "memory_plus": _memory_plus_from_exact_product}[target])
    with pytest.raises(AssertionError):
        pin()
