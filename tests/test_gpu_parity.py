"""GPU parity of the HIP path against the oracle, through the C ABI (needs an MI355X).

Small workloads are compared element by element over every token; the full-size
workloads (16M and 64M keys) run exactly as the benchmark does and are compared on
sampled tokens, which the oracle computes one by one.
"""

from __future__ import annotations

import gc
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle import pkm as O  # noqa: E402
from synth import CONFIGS  # noqa: E402
from synth import inputs as S  # noqa: E402
from tests import parity as PAR  # noqa: E402


def say(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _G():
    from tests import gpu_util
    return gpu_util


def _oracle_inputs(wl, rows=None):
    """float64 oracle views of the stored inputs (optionally a subset of tokens)."""
    cfg, dt = wl.cfg, wl.cfg.dtype
    x = O.to_f64(wl.inp["x"] if rows is None else wl.inp["x"][rows], dt)
    return x, O.to_f64(wl.inp["W_q"], dt), O.to_f64(wl.inp["subkeys"], dt)


def check_order_valid(idx, score, what):
    """Each GPU list is sorted by score desc, and by index asc among exactly equal scores."""
    s = score.reshape(-1, score.shape[-1]).astype(np.float64)
    i = idx.reshape(s.shape).astype(np.int64)
    assert (np.diff(s, axis=1) <= 0).all(), f"{what}: scores not non-increasing"
    eq = np.diff(s, axis=1) == 0
    assert (np.diff(i, axis=1)[eq] > 0).all(), f"{what}: equal scores not in ascending index order"


def table_rows(wl, needed, n_check=256):
    """``rows_of`` over the value rows in `needed`, copied out of the device table in one gather.

    The table is an input: the seeded device generator filled it.  A random sample of the
    copied rows is compared bitwise with the host generator's rows before they are used.
    """
    G = _G()
    uniq = np.unique(np.asarray(needed, dtype=np.int64).ravel())
    host = G.to_host(wl.values.index_select(0, torch.from_numpy(uniq).to(wl.values.device)))
    pick = np.random.default_rng(len(uniq)).choice(len(uniq), min(n_check, len(uniq)), replace=False)
    np.testing.assert_array_equal(host[pick], wl.host_rows(uniq[pick]))
    dt = wl.cfg.dtype
    return lambda r: O.to_f64(host[np.searchsorted(uniq, np.asarray(r, dtype=np.int64))], dt)


def full_check(wl, o, rows=None, e2e_rows=None):
    """Stage-wise parity of one debug forward `o` (numpy dict) on the token subset `rows`, and
    end-to-end parity on `e2e_rows` (a subset of `rows`; default: all of them)."""
    cfg, dt = wl.cfg, wl.cfg.dtype
    G = _G()
    tok = np.arange(wl.T) if rows is None else np.asarray(rows)
    x, Wq, K = _oracle_inputs(wl, tok)
    # a1-a2: normalised query
    q1o, q2o = O.normalized_query(x, Wq, cfg.H, cfg.d_q, cfg.qk_norm, cfg.norm_eps, dt)
    qg = o["qhat"][tok]
    khat_dev = torch.empty((cfg.H, 2, cfg.n_sub, cfg.d_h), dtype=G.TORCH_DT[dt], device="cuda")
    import sparse_key_value_amd as P
    P.pkm_copy_normalized_subkeys(wl.pkm.handle, khat_dev)
    torch.cuda.synchronize()
    kg = G.to_host(khat_dev)
    K1o, K2o = O.normalized_subkeys(K, cfg.qk_norm, cfg.norm_eps, dt)
    if dt == "bf16":
        # q = x W_q is stored in bf16 before the norm reads it, and q-hat is rounded again.  Each
        # bf16 rounding moves a value by at most 2^-8 of itself, and so can the RMS of the rounded
        # row: at most 3 * 2^-8 of the exact float64 chain in all, and one ulp of a value is at
        # least 2^-8 of it, so three ulps.  The oracle rounds at the same two places, so the two
        # agree bit for bit except where the GPU's fp32 product and the exact one lie on either
        # side of a bf16 rounding boundary
        qn = O.project_query(x, Wq, cfg.H, cfg.d_q)
        qn = O.rmsnorm(qn, cfg.norm_eps) if cfg.qk_norm else qn
        PAR.check_bf16_rounded(qg, qn.reshape(qg.shape), 2e-5, "qhat", ulps=3.0)
        same = float((O.bf16_bits_to_f64(qg) == np.concatenate([q1o, q2o], axis=-1).reshape(qg.shape)).mean())
        assert same >= 0.99, f"qhat equals the oracle's in only {same:.5f} of its elements"
        say(f"{cfg.name}: qhat equal to the oracle's in {same:.5f} of its elements")
        Kn = O.rmsnorm(K, cfg.norm_eps) if cfg.qk_norm else K
        PAR.check_bf16_rounded(kg, Kn, 1e-6, "normalised sub-keys")
    else:
        # fp32 sums of d_model products: their rounding error grows about as sqrt(d_model)
        # (the kernel's fma order emulated on the CPU at d_model = 65,536 leaves up to 1.7e-5 on
        # q-hat); widths up to 256 keep the plain tolerance
        g = max(1.0, float(np.sqrt(cfg.d_model / 256)))
        qo = np.concatenate([q1o, q2o], axis=-1).reshape(qg.shape)
        np.testing.assert_allclose(qg, qo, rtol=2e-5 * g, atol=2e-6 * g)
        np.testing.assert_allclose(kg, np.stack([K1o, K2o], axis=1), rtol=2e-5, atol=2e-6)

    # a3-a6 stage-wise: the oracle selects from the GPU's own qhat and khat bytes
    qgf = O.to_f64(qg, dt).reshape(len(tok), cfg.H, cfg.d_q)
    q1g, q2g = qgf[..., :cfg.d_h], qgf[..., cfg.d_h:]
    kgf = O.to_f64(kg, dt)
    K1g, K2g = kgf[:, 0], kgf[:, 1]
    sel = O.select(q1g, q2g, K1g, K2g, cfg.k)
    hidx, hsc = o["half_idx"][tok], o["half_score"][tok]
    check_order_valid(hidx, hsc, "per-half lists")
    ex_h = PAR.check_lists(hidx, sel["half_idx"], sel["half_score"],
                           PAR.half_choice_scores(q1g, q2g, K1g, K2g, hidx), "per-half top-k")
    gidx, gsc, gw = o["idx"][tok], o["score"][tok], o["w"][tok]
    check_order_valid(gidx, gsc, "final lists")
    ex_f = PAR.check_lists(gidx, sel["idx"], sel["score"], PAR.cell_choice_scores(q1g, q2g, K1g, K2g, gidx),
                           "final top-k")
    np.testing.assert_allclose(gw.sum(axis=-1), 1.0, atol=1e-5)
    assert (gw > 0).all() and (np.diff(gw, axis=-1) <= 1e-7).all()
    # GPU weights vs softmax of the GPU's own scores (float64)
    np.testing.assert_allclose(gw, O.softmax(gsc.astype(np.float64)), rtol=2e-6, atol=1e-7)

    # a7 stage-wise: oracle gather of the GPU's indices and weights
    rows_of = table_rows(wl, gidx)
    y_st = O.weighted_bag(rows_of, gidx.astype(np.int64), gw.astype(np.float64))
    PAR.check_rows(o["y"][tok], y_st, 1e-4, "gather (stage)")

    # a8 stage-wise: gate from the GPU's y
    if cfg.memory_plus:
        out_st = O.memory_plus(o["y"][tok].astype(np.float64), x, O.to_f64(wl.inp["W1"], dt),
                               O.to_f64(wl.inp["W2"], dt), dt)
        PAR.check_rows(O.to_f64(o["out"][tok], dt), out_st, PAR.TOL[dt], "Memory+ gate (stage)")

    # end to end from x: the oracle's own q, khat; indices under the near-tie rule, outputs re-evaluated
    if e2e_rows is not None:
        sub = np.searchsorted(tok, np.asarray(e2e_rows))
        assert (tok[sub] == np.asarray(e2e_rows)).all(), "e2e_rows must be a subset of rows"
        tok, x, q1o, q2o, gidx = tok[sub], x[sub], q1o[sub], q2o[sub], gidx[sub]
    ora = O.select(q1o, q2o, K1o, K2o, cfg.k)
    tau_scale = 1.0 if dt == "f32" else 100.0   # bf16: qhat may round the other way (about 4e-3 in a score)
    old = PAR.TAU
    PAR.TAU = old * tau_scale
    try:
        ex_e = PAR.check_lists(gidx, ora["idx"], ora["score"], PAR.cell_choice_scores(q1o, q2o, K1o, K2o, gidx),
                               "end-to-end top-k")
    finally:
        PAR.TAU = old
    y_ref, _ = PAR.reference_on_gpu_choice(q1o, q2o, K1o, K2o, gidx, rows_of)
    out_ref = (O.memory_plus(y_ref, x, O.to_f64(wl.inp["W1"], dt), O.to_f64(wl.inp["W2"], dt), dt)
               if cfg.memory_plus else y_ref)
    rel = PAR.check_rows(O.to_f64(o["out"][tok], dt), out_ref, PAR.TOL[dt], "output (end to end)")
    say(f"{cfg.name}: stage-wise on {len(gsc)} tokens: excused per-half {ex_h}, final {ex_f}; end to end on "
        f"{len(tok)} tokens: excused {ex_e}, worst out rel err {rel:.2e}")
    return ex_e


def run_debug(wl):
    o = wl.forward_debug()
    return {k: _G().to_host(v) for k, v in o.items()}


# ----------------------------------------------------------------------------------


def test_device_value_generator_is_bit_identical_to_host():
    G = _G()
    from synth import device as SD
    for dt, d_v in (("bf16", 1024), ("f32", 256), ("bf16", 136)):
        say(f"value generator {dt} d_v={d_v}")
        t = torch.empty((4096, d_v), dtype=G.TORCH_DT[dt], device="cuda")
        SD.fill_values(t, seed=11)
        host = S.value_rows(11, np.arange(4096), d_v, dt)
        np.testing.assert_array_equal(G.to_host(t), host)
    # rows far into a 64M-row table (the counter row * d_v + col crosses 2^36): the kernel is given the
    # address row 0 would have, and writes only rows [row0, row0 + 64), which are exactly the tensor `t`
    t = torch.empty((64, 1024), dtype=torch.bfloat16, device="cuda")
    row0 = (1 << 26) - 64
    rc = SD._lib.synth_fill_values(t.data_ptr() - row0 * 1024 * 2, row0, 64, 1024, 1, 0,
                                   torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(G.to_host(t), S.value_rows(0, np.arange(row0, row0 + 64), 1024, "bf16"))


@pytest.mark.parametrize("dt,dim,n_rows,n_bags,bag", [
    ("bf16", 2048, 5000, 37, 128), ("bf16", 1024, 3000, 130, 33), ("f32", 256, 4000, 65, 32),
    ("bf16", 64, 700, 300, 5), ("f32", 12, 99, 17, 3), ("bf16", 4096, 257, 9, 16),
    ("bf16", 256, 6000, 80, 128),     # one GPU's column shard of the 2048-wide table over 8 GPUs
])
def test_embedding_bag_matches_oracle(dt, dim, n_rows, n_bags, bag):
    import sparse_key_value_amd as P
    G = _G()
    say(f"embedding_bag {dt} dim={dim} rows={n_rows} bags={n_bags}x{bag}")
    rng = np.random.default_rng([dim, n_bags])
    table = S.value_rows(5, np.arange(n_rows), dim, dt)
    idx = rng.integers(0, n_rows, (n_bags, bag)).astype(np.int32)
    idx[0, 0] = idx[0, -1]            # a duplicate in a bag counts twice
    idx[-1, 0] = -3                   # out-of-range indices contribute nothing
    idx[-1, -1] = n_rows
    w = rng.standard_normal((n_bags, bag)).astype(np.float32)
    y = torch.empty((n_bags, dim), dtype=torch.float32, device="cuda")
    P.pkm_embedding_bag(G.to_dev(table, dt), n_rows, dim, dt, torch.from_numpy(idx).cuda(),
                        torch.from_numpy(w).cuda(), n_bags, bag, y)
    torch.cuda.synchronize()
    valid = (idx >= 0) & (idx < n_rows)
    tab = O.to_f64(table, dt)
    ref = O.weighted_bag(lambda r: tab[r], np.where(valid, idx, 0).astype(np.int64)[:, None, :],
                         np.where(valid, w, 0.0).astype(np.float64)[:, None, :])
    PAR.check_rows(G.to_host(y), ref, 1e-5, "embedding bag")
    # n_bags = 0 is a no-op
    P.pkm_embedding_bag(G.to_dev(table, dt), n_rows, dim, dt, torch.from_numpy(idx).cuda(),
                        torch.from_numpy(w).cuda(), 0, bag, y)


def test_tiny_fp32_end_to_end_all_tokens():
    cfg = CONFIGS["tiny_fp32_65k"]
    say(f"{cfg.name} T={cfg.T}")
    wl = _G().Workload(cfg)
    o = run_debug(wl)
    full_check(wl, o)
    wl.close()


@pytest.mark.parametrize("T", [1, 7, 129, 509])
def test_tiny_fp32_ragged_token_counts(T):
    cfg = CONFIGS["tiny_fp32_65k"]
    say(f"{cfg.name} T={T}")
    wl = _G().Workload(cfg, T=T, max_tokens=512)
    o = run_debug(wl)
    full_check(wl, o)
    wl.close()


@pytest.mark.timeout(600)
def test_fp32_batch_with_more_token_tiles_than_a_grid_row():
    """An fp32 gated batch of 65,537 * 64 tokens: its two fp32 GEMMs have one more 64-token tile
    than a launch grid's y dimension holds (65,536), so the tiles run along x.  Narrow widths keep
    it small; properties on every token, the oracle on the first and last tiles and random tokens."""
    T = 65537 * 64
    cfg = CONFIGS["tiny_fp32_65k"].with_(name="fp32_4m_tokens", T=T, d_model=16, H=1, d_q=8, n_sub=16, k=4,
                                         d_v=16, qk_norm=True, memory_plus=True)
    say(f"fp32 T={T}")
    wl = _G().Workload(cfg)
    o = run_debug(wl)
    assert o["idx"].shape == (T, 1, 4) and o["out"].shape == (T, 16)
    assert (o["idx"] >= 0).all() and (o["idx"] < cfg.N).all()
    np.testing.assert_allclose(o["w"].sum(axis=-1), 1.0, atol=1e-5)
    check_order_valid(o["idx"], o["score"], "final lists (all tokens)")
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(T - 64, T), rng.choice(T, 128, replace=False)]))
    full_check(wl, o, rows=rows)
    wl.close()
    del wl, o
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d_model,d_v,gate", [(65536, 32, True), (32, 65536, False)])
def test_widest_model_and_value_rows(dt, d_model, d_v, gate):
    """d_model and d_value at the largest width the boundary accepts (65,536): the weight
    transposes at create, the GEMMs over 65,536-wide operands, and value rows of 128 or 256 KiB
    gathered in 32 or 64 column blocks; every token against the oracle."""
    base = CONFIGS["pkm_1m_bf16"] if dt == "bf16" else CONFIGS["tiny_fp32_65k"]
    cfg = base.with_(name=f"wide_{d_model}_{d_v}", T=64, d_model=d_model, H=1, d_q=8, n_sub=8, k=4, d_v=d_v,
                     qk_norm=True, memory_plus=gate)
    say(f"{dt} d_model={d_model} d_value={d_v} gate={gate}")
    wl = _G().Workload(cfg, seed=3)
    o = run_debug(wl)
    full_check(wl, o)
    wl.close()


@pytest.mark.timeout(600)
def test_largest_accepted_batch_of_selection_rows():
    """max_tokens * n_heads = 2^24, the most the boundary accepts: 2^22 tokens of 4 heads, so the
    selection runs over 2^25 (token, head, half) rows (2^31 work-items in the one-wave-per-row
    launches) and the combine over 2^24.  Narrow widths keep it small (54 GiB of workspace);
    properties on every token, the oracle on the first and last scoring blocks and random tokens."""
    T = 1 << 22
    cfg = CONFIGS["pkm_1m_bf16"].with_(name="bf16_max_rows", T=T, d_model=32, H=4, d_q=8, n_sub=64, k=4, d_v=16)
    say(f"bf16 T={T} H=4: 2^25 selection rows")
    wl = _G().Workload(cfg)
    o = run_debug(wl)
    assert o["idx"].shape == (T, 4, 4)
    assert (o["idx"] >= 0).all() and (o["idx"] < cfg.N).all()
    np.testing.assert_allclose(o["w"].sum(axis=-1), 1.0, atol=1e-5)
    check_order_valid(o["idx"], o["score"], "final lists (all tokens)")
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([np.arange(512), np.arange(T - 512, T), rng.choice(T, 256, replace=False)]))
    full_check(wl, o, rows=rows)
    wl.close()
    del wl, o
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,T", [("memplus_16m_bf16", 200), ("memplus_64m_bf16", 77),
                                    ("memplus_16m_bf16", 1), ("memplus_64m_bf16", 1)])
def test_small_batches_split_the_sub_keys(name, T):
    """A batch far smaller than the chip (200 and 77 tokens over 4,096 and 8,192 sub-keys, and a
    single token, whose one valid lane per wave fragment meets every split): every block sweeps
    one range of the sub-keys and the ranges share each row's candidate list through atomic
    counts."""
    cfg = CONFIGS[name].with_(T=T)
    say(f"{name} T={T}: sub-key splits")
    wl = _G().Workload(cfg, T=T)
    o = run_debug(wl)
    full_check(wl, o)
    wl.close()
    del wl, o
    gc.collect()
    torch.cuda.empty_cache()


def test_pkm_1m_bf16_stagewise_ragged():
    cfg = CONFIGS["pkm_1m_bf16"]
    say(f"{cfg.name} T=300")
    wl = _G().Workload(cfg, T=300)
    o = run_debug(wl)
    full_check(wl, o)
    wl.close()


@pytest.mark.parametrize("case", [
    dict(name="figD_n8_k2", n_sub=8, k=2, H=1, d_q=128, d_model=64, d_v=64, T=40),
    dict(name="n100_k5_h3", n_sub=100, k=5, H=3, d_q=256, d_model=128, d_v=128, T=200),
    dict(name="k1", n_sub=64, k=1, H=2, d_q=128, d_model=64, d_v=64, T=70),
    dict(name="d_h128_gate", n_sub=200, k=32, H=2, d_q=256, d_model=256, d_v=128, T=131, memory_plus=True),
    dict(name="n33_k32", n_sub=33, k=32, H=1, d_q=128, d_model=64, d_v=64, T=64),
    dict(name="n1_k1", n_sub=1, k=1, H=2, d_q=128, d_model=64, d_v=64, T=17),        # one key: N = 1
    dict(name="n32_k32", n_sub=32, k=32, H=1, d_q=128, d_model=64, d_v=64, T=40),    # k = n_sub
    dict(name="h64", n_sub=64, k=4, H=64, d_q=128, d_model=64, d_v=64, T=33),        # the most heads
])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_edge_shapes(case, dt):
    case = dict(case)
    name = case.pop("name")
    cfg = CONFIGS["pkm_1m_bf16"].with_(name=f"{name}_{dt}", dtype=dt, qk_norm=(dt == "bf16"),
                                        memory_plus=case.pop("memory_plus", False), **case)
    say(f"edge {cfg.name}")
    wl = _G().Workload(cfg, seed=3)
    o = run_debug(wl)
    full_check(wl, o)
    wl.close()


@pytest.mark.parametrize("case", [
    # bf16 without qk-norm; 96-wide values (12 slices of 16 bytes: lanes not a multiple of 64)
    dict(name="bf16_no_norm_dv96", dtype="bf16", qk_norm=False, n_sub=128, k=16, H=2, d_q=256, d_model=128, d_v=96,
         T=90),
    # fp32 with qk-norm and the gate
    dict(name="f32_norm_gate", dtype="f32", qk_norm=True, memory_plus=True, n_sub=150, k=8, H=3, d_q=128, d_model=96,
         d_v=96, T=77),
    # eight heads, gated bf16
    dict(name="h8_gate", dtype="bf16", qk_norm=True, memory_plus=True, n_sub=256, k=32, H=8, d_q=128, d_model=256,
         d_v=256, T=65),
    # 256-wide sub-keys (the 16M-key kernels) with a partial last chunk of sub-keys
    dict(name="dh256_partial_chunk", dtype="bf16", qk_norm=True, n_sub=77, k=8, H=2, d_q=512, d_model=128, d_v=64,
         T=70),
    # gated, with z rows off 16-byte alignment (the gate reads z in 4-byte loads): bf16 z at
    # byte 12 of a 140-byte row, fp32 z at byte 24 of a 56-byte row
    dict(name="bf16_gate_z_unaligned", dtype="bf16", qk_norm=True, memory_plus=True, n_sub=96, k=8, H=1, d_q=6,
         d_model=64, d_v=64, T=50),
    dict(name="f32_gate_z_unaligned", dtype="f32", qk_norm=True, memory_plus=True, n_sub=96, k=8, H=3, d_q=2,
         d_model=64, d_v=8, T=50),
])
def test_flag_combinations(case):
    case = dict(case)
    name = case.pop("name")
    cfg = CONFIGS["pkm_1m_bf16"].with_(name=name, memory_plus=case.pop("memory_plus", False), **case)
    say(f"flags {cfg.name}")
    wl = _G().Workload(cfg, seed=7)
    full_check(wl, run_debug(wl))
    wl.close()


def _sample_tokens(T, n=96, tail=24):
    """About n evenly spread tokens plus the last `tail` (the ragged last block)."""
    return np.unique(np.concatenate([np.linspace(0, T - 1, n).astype(np.int64), np.arange(max(0, T - tail), T)]))


@pytest.mark.parametrize("case", [
    # batches that give every CU an 8-wave scoring block (512 tokens x one (head, half) each),
    # with a ragged last block and a partial last chunk of
    # sub-keys: 256-, 128- and 64-wide sub-keys.  The GPU runs every token; the oracle
    # checks a spread of tokens over both wave groups and the end of the last block.
    dict(name="eight_waves_dh256", dtype="bf16", qk_norm=True, n_sub=1100, k=8, H=64, d_q=512, d_model=64, d_v=64,
         T=600),
    dict(name="eight_waves_dh128", dtype="bf16", qk_norm=True, memory_plus=True, n_sub=1030, k=16, H=16, d_q=256,
         d_model=128, d_v=128, T=3700),
    # more blocks than CUs (10 token tiles x 32 head halves = 320 blocks), ragged last tile
    dict(name="eight_waves_320_blocks", dtype="bf16", qk_norm=True, n_sub=1030, k=16, H=16, d_q=256, d_model=128,
         d_v=128, T=5000),
    dict(name="eight_waves_f32_dh64", dtype="f32", qk_norm=False, n_sub=1050, k=8, H=32, d_q=128, d_model=64, d_v=64,
         T=1600),
    dict(name="eight_waves_f32_dh128", dtype="f32", qk_norm=True, memory_plus=True, n_sub=1100, k=32, H=32, d_q=256,
         d_model=64, d_v=64, T=1600),
    # groups of 8 sub-keys (four group maxima per chunk) in 8-wave blocks
    dict(name="eight_waves_groups_of_8", dtype="bf16", qk_norm=True, n_sub=700, k=16, H=64, d_q=512, d_model=64,
         d_v=64, T=700),
    # batches that fill the CUs only with 32-token waves (8-wave blocks of 256 tokens)
    dict(name="eight_waves_32_tokens_dh256", dtype="bf16", qk_norm=True, n_sub=1100, k=8, H=64, d_q=512, d_model=64,
         d_v=64, T=300),
    dict(name="eight_waves_32_tokens_dh128", dtype="bf16", qk_norm=True, memory_plus=True, n_sub=1030, k=16, H=16,
         d_q=256, d_model=128, d_v=128, T=1900),
    dict(name="eight_waves_32_tokens_f32_dh64", dtype="f32", qk_norm=False, n_sub=1050, k=8, H=32, d_q=128, d_model=64,
         d_v=64, T=1000),
])
def test_eight_wave_scoring_blocks(case):
    case = dict(case)
    name = case.pop("name")
    cfg = CONFIGS["pkm_1m_bf16"].with_(name=name, memory_plus=case.pop("memory_plus", False), **case)
    say(f"8-wave scoring {cfg.name}")
    wl = _G().Workload(cfg, seed=7)
    o = run_debug(wl)
    T = cfg.T
    full_check(wl, o, rows=_sample_tokens(T))
    wl.close()


@pytest.mark.parametrize("dt,H,T,n_sub,d_q,k", [("f32", 2, 100, 96, 128, 16), ("bf16", 2, 100, 96, 128, 16),
                                                # 64 heads x 520 tokens over 1,040 sub-keys: 8-wave scoring
                                                # blocks with a ragged last block
                                                ("bf16", 64, 520, 1040, 128, 16),
                                                # split sub-key ranges: the zero tokens tie k times per lane
                                                # and range, more than a lane's LDS stash holds (64-, 256-wide
                                                # bf16 and 64-wide fp32 sub-keys), and every such row
                                                # overflows into the exhaustive pass
                                                ("bf16", 4, 100, 1040, 128, 16), ("bf16", 4, 200, 1040, 512, 16),
                                                ("f32", 4, 100, 1040, 128, 16),
                                                # k > 32: the two MFMA passes (8-wave blocks), the split
                                                # ranges and the exhaustive rows, 64-key lane lists
                                                ("bf16", 64, 520, 1024, 128, 64), ("bf16", 4, 100, 2048, 512, 48),
                                                ("f32", 2, 100, 96, 128, 40)])
def test_exact_ties_resolve_to_lowest_index(dt, H, T, n_sub, d_q, k):
    """Duplicated sub-keys give bitwise-equal scores; zero tokens give all-zero scores."""
    cfg = CONFIGS["pkm_1m_bf16"].with_(name=f"ties_{dt}_h{H}_k{k}", dtype=dt, n_sub=n_sub, k=k, H=H, d_q=d_q,
                                        d_model=64, d_v=64, T=T, qk_norm=True)
    inp = S.make_inputs(cfg, seed=4)
    sk = inp["subkeys"].copy()
    sk[:, :, 1::2] = sk[:, :, 0::2]      # sub-key 2i+1 duplicates 2i in every codebook
    inp["subkeys"] = sk
    x = inp["x"].copy()
    x[::5] = 0                          # every fifth token is all zero: every score is 0
    inp["x"] = x
    say(f"ties {dt} H={H} T={T} n_sub={n_sub} d_q={d_q} k={k}")
    wl = _G().Workload(cfg, seed=4, host_inputs=inp)
    o = run_debug(wl)
    # the oracle on every token of the small cases, on a spread (every fifth token, the zero
    # ones, included) of the 64-head one
    full_check(wl, o, rows=None if H < 64 else np.unique(np.concatenate([_sample_tokens(T), np.arange(0, T, 5)])))
    # zero tokens: per-half lists are 0..k-1 and the final list is cells (0, 0..k-1)
    z = np.arange(0, cfg.T, 5)
    assert (o["half_idx"][z] == np.arange(cfg.k)).all()
    assert (o["idx"][z] == np.arange(cfg.k)).all()
    np.testing.assert_allclose(o["w"][z], 1.0 / cfg.k, rtol=1e-6)
    # duplicated sub-keys: whenever both of a pair are listed, the even one comes first
    for lst in (o["half_idx"],):
        l = lst.reshape(-1, cfg.k)
        pos = {}
        for r in range(l.shape[0]):
            p = {int(v): j for j, v in enumerate(l[r])}
            for v, j in p.items():
                if v % 2 == 1 and (v - 1) in p:
                    assert p[v - 1] < j
    wl.close()


@pytest.mark.parametrize("n_sub", [256, 1100])   # exhaustive rows; split sub-key ranges with atomic counts
def test_forward_is_deterministic_and_matches_plain_forward(n_sub):
    import sparse_key_value_amd as P
    cfg = CONFIGS["pkm_1m_bf16"].with_(n_sub=n_sub, T=257, d_v=256)
    say(f"determinism n_sub={n_sub}")
    wl = _G().Workload(cfg, seed=8)
    outs = []
    for _ in range(2):
        out = torch.empty((wl.T, cfg.d_out), dtype=torch.bfloat16, device="cuda")
        idx = torch.empty((wl.T, cfg.H, cfg.k), dtype=torch.int32, device="cuda")
        w = torch.empty((wl.T, cfg.H, cfg.k), dtype=torch.float32, device="cuda")
        P.pkm_forward(wl.pkm.handle, wl.dev["x"], wl.T, out, idx, w)
        torch.cuda.synchronize()
        outs.append((out.view(torch.int16).cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()))
    dbg = run_debug(wl)
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(outs[0][1], dbg["idx"])
    np.testing.assert_array_equal(outs[0][2], dbg["w"])
    np.testing.assert_array_equal(outs[0][0], dbg["out"].view(np.int16))
    # T = 0 enqueues nothing and succeeds
    P.pkm_forward(wl.pkm.handle, wl.dev["x"], 0, out)
    with pytest.raises(P.PkmError):
        P.pkm_forward(wl.pkm.handle, wl.dev["x"], wl.T + 1, out)
    wl.close()


def test_many_batch_sizes_rebuild_their_gemm_plans_alike():
    """Batch sizes 1 to 80 in one process, both bf16 products (projection and gate) per forward:
    more exact shapes than the library's plan cache keeps (64), so the first ones are evicted and
    built again.  A rebuilt plan takes its power-of-two bucket's algorithm again, so batch sizes
    run before and after the evictions give the same bits; the last batch agrees with the oracle."""
    import sparse_key_value_amd as P
    cfg = CONFIGS["pkm_1m_bf16"].with_(n_sub=256, T=80, d_v=256, memory_plus=True, d_model=256)
    say("gemm plans over batch sizes 1-80")
    wl = _G().Workload(cfg, seed=12)

    def fwd(T):
        out = torch.empty((T, cfg.d_out), dtype=torch.bfloat16, device="cuda")
        idx = torch.empty((T, cfg.H, cfg.k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, cfg.H, cfg.k), dtype=torch.float32, device="cuda")
        P.pkm_forward(wl.pkm.handle, wl.dev["x"], T, out, idx, w)
        torch.cuda.synchronize()
        return out.view(torch.int16).cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()

    first = {T: fwd(T) for T in (3, 37, 64)}
    for T in range(1, 81):
        fwd(T)
    for T, ref in first.items():
        for a, b in zip(ref, fwd(T)):
            np.testing.assert_array_equal(a, b)
    full_check(wl, run_debug(wl))
    wl.close()


def test_concurrent_forwards_share_the_gemm_plans():
    """Two host threads, each with its own handle and stream, run forwards over 70 batch sizes
    at once (both bf16 products per forward): they share the library's GEMM plans, whose
    cache evicts entries while the other thread may be launching with them.  Every result
    equals the same forward run alone afterwards, bit for bit."""
    import threading

    import sparse_key_value_amd as P
    cfg = CONFIGS["pkm_1m_bf16"].with_(n_sub=256, T=96, d_v=256, memory_plus=True, d_model=256)
    say("concurrent forwards over batch sizes")
    wls = [_G().Workload(cfg, seed=s) for s in (21, 22)]
    sizes = [list(range(1, 71)), list(range(96, 26, -1))]

    def fwd(wl, T, stream):
        out = torch.empty((T, cfg.d_out), dtype=torch.bfloat16, device="cuda")
        idx = torch.empty((T, cfg.H, cfg.k), dtype=torch.int32, device="cuda")
        P.pkm_forward(wl.pkm.handle, wl.dev["x"], T, out, idx, None, stream=stream)
        stream.synchronize()
        return out.view(torch.int16).cpu().numpy(), idx.cpu().numpy()

    got = [{}, {}]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            for T in sizes[i]:
                got[i][T] = fwd(wls[i], T, s)
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    s = torch.cuda.Stream()
    for i in range(2):
        for T in sizes[i]:
            for a, b in zip(got[i][T], fwd(wls[i], T, s)):
                np.testing.assert_array_equal(a, b)
    for wl in wls:
        wl.close()


def test_forward_on_a_side_stream_follows_its_inputs():
    """The forward enqueues every kernel (hipBLASLt's included) on the caller's stream: on a
    side stream whose input is written late by earlier work on that same stream, the result
    equals the default stream's bit for bit (a kernel on any other stream would read the
    input before it is written)."""
    import sparse_key_value_amd as P
    cfg = CONFIGS["pkm_1m_bf16"].with_(n_sub=1100, T=700, d_v=256)
    say("side stream")
    wl = _G().Workload(cfg, seed=9)
    x = wl.dev["x"]

    def buffers():
        return (torch.empty((wl.T, cfg.d_out), dtype=torch.bfloat16, device="cuda"),
                torch.empty((wl.T, cfg.H, cfg.k), dtype=torch.int32, device="cuda"),
                torch.empty((wl.T, cfg.H, cfg.k), dtype=torch.float32, device="cuda"))

    ref = buffers()
    P.pkm_forward(wl.pkm.handle, x, wl.T, *ref)
    torch.cuda.synchronize()
    ref = [r.view(torch.int16).cpu() if r.dtype == torch.bfloat16 else r.cpu() for r in ref]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    got = []
    for explicit in (False, True):
        with torch.cuda.stream(s):
            a = torch.randn(4096, 4096, device="cuda")
            for _ in range(8):   # about a millisecond of work ahead of the input's copy
                a = torch.tanh(a @ a)
            x2 = torch.zeros_like(x)
            x2.copy_(x)
            bufs = buffers()
        if explicit:   # the stream passed by argument, from outside its context
            P.pkm_forward(wl.pkm.handle, x2, wl.T, *bufs, stream=s)
        else:          # the current stream
            with torch.cuda.stream(s):
                P.pkm_forward(wl.pkm.handle, x2, wl.T, *bufs)
        s.synchronize()
        got.append([b.view(torch.int16).cpu() if b.dtype == torch.bfloat16 else b.cpu() for b in bufs])
    for g in got:
        for r, b in zip(ref, g):
            assert torch.equal(r, b)
    wl.close()


def _sample_rows(T, n=40, seed=1):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 1, T - 1], rng.choice(T, n, replace=False)]))
    return rows


def _benchmark_block_rows(T, n_random=272, seed=1):
    """The first 512-token scoring block (both groups of four waves), the last 256 tokens (the end
    of the last block) and random tokens: 1,024 tokens in all at 16,384 tokens."""
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(min(512, T)), np.arange(max(0, T - 256), T),
                                     rng.choice(T, n_random, replace=False)]))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,seed", [("memplus_16m_bf16", 0), ("memplus_64m_bf16", 0), ("pkm_1m_bf16", 0),
                                       ("memplus_16m_bf16", 1)])
def test_full_size_as_benchmarked(name, seed):
    """The headline, the largest and the 1M-key workload at full size, run exactly as the
    benchmark runs them (the headline also on a second seed: other inputs, weights and table).
    Properties on every token; the oracle on 1,024 tokens of the 16M- and 64M-key batches (a
    whole 512-token scoring block, the end of the last block and random tokens), and stage-wise
    on all 8,192 tokens of the 1M-key batch (which takes the 32-token waves of the scoring
    passes) with end to end on a sample."""
    cfg = CONFIGS[name]
    say(f"{name} seed {seed}: filling {cfg.N} x {cfg.d_v} value table on the GPU")
    wl = _G().Workload(cfg, seed=seed)
    say(f"{name}: forward T={cfg.T}")
    o = run_debug(wl)
    # the entry point the benchmark times (no debug outputs) returns the debug forward's
    # results bit for bit, so the oracle checks below hold for it too
    import sparse_key_value_amd as P
    plain = (torch.empty((cfg.T, cfg.d_out), dtype=_G().TORCH_DT[cfg.dtype], device="cuda"),
             torch.empty((cfg.T, cfg.H, cfg.k), dtype=torch.int32, device="cuda"),
             torch.empty((cfg.T, cfg.H, cfg.k), dtype=torch.float32, device="cuda"))
    P.pkm_forward(wl.pkm.handle, wl.dev["x"], cfg.T, *plain)
    torch.cuda.synchronize()
    for key, t in zip(("out", "idx", "w"), plain):
        np.testing.assert_array_equal(_G().to_host(t), o[key], err_msg=f"{name}: plain forward {key}")
    del plain
    # properties over every token
    assert (o["idx"] >= 0).all() and (o["idx"] < cfg.N).all()
    np.testing.assert_allclose(o["w"].sum(axis=-1), 1.0, atol=1e-5)
    check_order_valid(o["idx"], o["score"], "final lists (all tokens)")
    if cfg.T <= 8192:
        rows, e2e = None, _sample_rows(cfg.T)
    else:
        rows, e2e = _benchmark_block_rows(cfg.T, seed=1 + seed), None
    say(f"{name}: oracle stage-wise on {cfg.T if rows is None else len(rows)} tokens")
    full_check(wl, o, rows=rows, e2e_rows=e2e)
    wl.close()
    del wl, o
    gc.collect()
    torch.cuda.empty_cache()


def test_combine_rounding_tie_takes_exhaustive_path():
    """fp32 sums that round to the same value reorder by flat index off the staircase.

    Half 0 scores: sub-key 10 -> 2^25, sub-key 3 -> 2^25 - 2; half 1: sub-key 20 -> 1.5,
    sub-key 7 -> 1.25 (every other sub-key -1000).  All four sums of the top-2 x top-2
    pairs round to 2^25 in fp32, so by flat index (a * 64 + b) the top-2 cells are
    3*64+7 = 199 and 3*64+20 = 212; (1,1) lies off the staircase (i+1)(j+1) <= 2, which
    the exhaustive path must catch.  The float64 oracle orders them by the exact sums;
    the two answers differ only inside the near-tie margin.
    """
    import sparse_key_value_amd as P
    n, dh = 64, 64
    K = np.full((1, 2, n, dh), 0.0, dtype=np.float32)
    K[0, :, :, 0] = -1000.0
    K[0, 0, 10, 0], K[0, 0, 3, 0] = 2.0 ** 25, 2.0 ** 25 - 2
    K[0, 1, 20, 0], K[0, 1, 7, 0] = 1.5, 1.25
    dev = torch.from_numpy(K).cuda()
    wq = torch.zeros((64, 128), dtype=torch.float32, device="cuda")
    vals = torch.zeros((n * n, 4), dtype=torch.float32, device="cuda")
    pk = P.ProductKeyMemory(d_model=64, n_heads=1, d_query=128, n_sub=n, k=2, d_value=4, dtype="f32", qk_norm=0,
                            memory_plus=0, max_tokens=4, W_q=wq, subkeys=dev, values=vals)
    q = np.zeros((1, 1, 2, dh), dtype=np.float32)
    q[0, 0, :, 0] = 1.0
    hi_ = torch.empty((1, 1, 2, 2), dtype=torch.int32, device="cuda")
    hs_ = torch.empty((1, 1, 2, 2), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, 1, 2), dtype=torch.int32, device="cuda")
    sc = torch.empty((1, 1, 2), dtype=torch.float32, device="cuda")
    w = torch.empty((1, 1, 2), dtype=torch.float32, device="cuda")
    P.pkm_select(pk.handle, torch.from_numpy(q).cuda(), 1, hi_, hs_, idx, sc, w)
    torch.cuda.synchronize()
    assert hi_.cpu().numpy().tolist() == [[[[10, 3], [20, 7]]]]
    assert idx.cpu().numpy().tolist() == [[[199, 212]]]
    assert sc.cpu().numpy().tolist() == [[[2.0 ** 25, 2.0 ** 25]]]
    np.testing.assert_allclose(w.cpu().numpy(), 0.5)
    # the oracle's float64 answer differs only within the near-tie margin
    q64 = q.astype(np.float64).reshape(1, 1, 2 * dh)
    sel = O.select(q64[..., :dh], q64[..., dh:], K[:, 0].astype(np.float64), K[:, 1].astype(np.float64), 2)
    assert sel["idx"].tolist() == [[[660, 647]]]
    ch = PAR.cell_choice_scores(q64[..., :dh], q64[..., dh:], K[:, 0].astype(np.float64), K[:, 1].astype(np.float64),
                                idx.cpu().numpy())
    PAR.check_lists(idx.cpu().numpy(), sel["idx"], sel["score"], ch, "rounding-tie case")
    pk.close()


@pytest.mark.parametrize("k", [32, 64])
def test_candidate_overflow_takes_exhaustive_path(k):
    """Scores rising with the sub-key index make the group-maximum bound loose.

    With s_i = i over 2,048 sub-keys in groups of 16, the k-th largest group maximum is
    2047 - 16 (k - 1) (1551 for k = 32), so about 500 (k = 64: 1,000) sub-keys reach the bound
    and overflow the candidate list; that row is then scored exhaustively.  Every score is
    an exact small integer, so the result must equal the oracle's exactly: per-half lists
    2047 .. 2048 - k, final cells by sum.
    """
    import sparse_key_value_amd as P
    n, dh = 2048, 64
    K = np.zeros((1, 2, n, dh), dtype=np.float32)
    K[0, 0, :, 0] = np.arange(n, dtype=np.float32)
    K[0, 1, :, 1] = np.arange(n, dtype=np.float32)[::-1] * 0.5   # half 1: best at low indices
    wq = torch.zeros((64, 128), dtype=torch.float32, device="cuda")
    vals = torch.zeros((n * n, 4), dtype=torch.float32, device="cuda")
    pk = P.ProductKeyMemory(d_model=64, n_heads=1, d_query=128, n_sub=n, k=k, d_value=4, dtype="f32", qk_norm=0,
                            memory_plus=0, max_tokens=8, W_q=wq, subkeys=torch.from_numpy(K).cuda(), values=vals)
    q = np.zeros((3, 1, 2, dh), dtype=np.float32)
    q[:, 0, 0, 0] = [1.0, 2.0, 0.5]
    q[:, 0, 1, 1] = [1.0, 1.0, 3.0]
    T = q.shape[0]
    hi_ = torch.empty((T, 1, 2, k), dtype=torch.int32, device="cuda")
    hs_ = torch.empty((T, 1, 2, k), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, 1, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((T, 1, k), dtype=torch.float32, device="cuda")
    w = torch.empty((T, 1, k), dtype=torch.float32, device="cuda")
    P.pkm_select(pk.handle, torch.from_numpy(q).cuda(), T, hi_, hs_, idx, sc, w)
    torch.cuda.synchronize()
    q64 = q.astype(np.float64).reshape(T, 1, 2 * dh)
    sel = O.select(q64[..., :dh], q64[..., dh:], K[:, 0].astype(np.float64), K[:, 1].astype(np.float64), k)
    assert (hi_.cpu().numpy()[:, 0, 0] == np.arange(n - 1, n - 1 - k, -1)).all()
    np.testing.assert_array_equal(hi_.cpu().numpy(), sel["half_idx"])
    np.testing.assert_array_equal(idx.cpu().numpy(), sel["idx"])
    np.testing.assert_allclose(sc.cpu().numpy(), sel["score"], rtol=0, atol=0)
    pk.close()


def test_candidate_overflow_in_eight_wave_blocks():
    """The overflow case above in every (token, head) of a batch that takes the 8-wave scoring
    blocks (64 heads x 600 tokens): each (token, head) gets one of the three queries, so its
    lists must equal the oracle's for that query exactly."""
    import sparse_key_value_amd as P
    n, dh, k, H, T = 2048, 64, 32, 64, 600
    K1 = np.zeros((2, n, dh), dtype=np.float32)
    K1[0, :, 0] = np.arange(n, dtype=np.float32)
    K1[1, :, 1] = np.arange(n, dtype=np.float32)[::-1] * 0.5
    K = np.ascontiguousarray(np.broadcast_to(K1, (H, 2, n, dh)))
    pats = np.zeros((3, 2, dh), dtype=np.float32)
    pats[:, 0, 0] = [1.0, 2.0, 0.5]
    pats[:, 1, 1] = [1.0, 1.0, 3.0]
    which = (np.arange(T)[:, None] + np.arange(H)[None, :]) % 3            # [T, H]
    q = np.ascontiguousarray(pats[which])                                  # [T, H, 2, dh]
    say(f"overflow in 8-wave blocks: T={T} H={H}")
    wq = torch.zeros((64, H * 2 * dh), dtype=torch.float32, device="cuda")
    vals = torch.zeros((n * n, 4), dtype=torch.float32, device="cuda")
    pk = P.ProductKeyMemory(d_model=64, n_heads=H, d_query=2 * dh, n_sub=n, k=k, d_value=4, dtype="f32", qk_norm=0,
                            memory_plus=0, max_tokens=T, W_q=wq, subkeys=torch.from_numpy(K).cuda(), values=vals)
    hi_ = torch.empty((T, H, 2, k), dtype=torch.int32, device="cuda")
    hs_ = torch.empty((T, H, 2, k), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, H, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((T, H, k), dtype=torch.float32, device="cuda")
    w = torch.empty((T, H, k), dtype=torch.float32, device="cuda")
    P.pkm_select(pk.handle, torch.from_numpy(q).cuda(), T, hi_, hs_, idx, sc, w)
    torch.cuda.synchronize()
    q64 = pats.astype(np.float64).reshape(3, 1, 2 * dh)
    sel = O.select(q64[..., :dh], q64[..., dh:], K1[None, 0].astype(np.float64), K1[None, 1].astype(np.float64), k)
    got_hi, got_idx, got_sc = hi_.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    for p in range(3):
        m = which == p
        np.testing.assert_array_equal(got_hi[m], np.broadcast_to(sel["half_idx"][p, 0], got_hi[m].shape))
        np.testing.assert_array_equal(got_idx[m], np.broadcast_to(sel["idx"][p, 0], got_idx[m].shape))
        np.testing.assert_array_equal(got_sc[m], np.broadcast_to(sel["score"][p, 0].astype(np.float32), got_sc[m].shape))
    pk.close()


def test_largest_sub_key_lists():
    """n_sub = 40,000 (the table would have 1.6e9 rows, near the int32 limit of the flat
    index): group maxima over 512 sub-keys, the largest group size built.  The selection
    (pkm_select) against the oracle's exhaustive per-half sort, exactly, since the scores
    are small multiples of 1/64."""
    import sparse_key_value_amd as P
    n, dh, k, T = 40000, 64, 32, 40
    rng = np.random.default_rng(11)
    K = (rng.integers(-64, 65, size=(1, 2, n, dh)) / 64.0).astype(np.float32)
    q = (rng.integers(-8, 9, size=(T, 1, 2, dh)) / 8.0).astype(np.float32)
    say(f"largest sub-key lists: n_sub={n}")
    wq = torch.zeros((64, 2 * dh), dtype=torch.float32, device="cuda")
    # pkm_select never reads the value table: the handle is made through the C ABI over a small
    # stand-in (ProductKeyMemory, made for forwards, insists on the whole 1.6e9-row table)
    vals = torch.zeros((16, 4), dtype=torch.float32, device="cuda")
    cfg = P.make_config(64, 1, 2 * dh, n, k, 4, "f32", 0, 0, T)
    ws = torch.empty(P.pkm_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    handle = P.pkm_create(cfg, wq, torch.from_numpy(K).cuda(), vals, None, None, ws, ws.numel())
    hi_ = torch.empty((T, 1, 2, k), dtype=torch.int32, device="cuda")
    hs_ = torch.empty((T, 1, 2, k), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, 1, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((T, 1, k), dtype=torch.float32, device="cuda")
    w = torch.empty((T, 1, k), dtype=torch.float32, device="cuda")
    P.pkm_select(handle, torch.from_numpy(q).cuda(), T, hi_, hs_, idx, sc, w)
    torch.cuda.synchronize()
    q64 = q.astype(np.float64).reshape(T, 1, 2 * dh)
    sel = O.select(q64[..., :dh], q64[..., dh:], K[:, 0].astype(np.float64), K[:, 1].astype(np.float64), k)
    np.testing.assert_array_equal(hi_.cpu().numpy(), sel["half_idx"])
    np.testing.assert_array_equal(idx.cpu().numpy(), sel["idx"])
    np.testing.assert_array_equal(sc.cpu().numpy(), sel["score"].astype(np.float32))
    P.pkm_destroy(handle)


@pytest.mark.parametrize("case", [
    # k > 32 (the pages' "about thirty" values, up to 64): the two MFMA passes with 256
    # candidate slots per row, the per-row exhaustive path, the wide combine
    dict(name="k33_two_pass", dtype="bf16", qk_norm=True, n_sub=1100, k=33, H=4, d_q=256, d_model=128, d_v=128, T=300),
    dict(name="k48_exhaustive_rows", dtype="bf16", qk_norm=True, n_sub=300, k=48, H=2, d_q=128, d_model=64, d_v=64,
         T=150),
    dict(name="k64_eight_waves", dtype="bf16", qk_norm=True, n_sub=2048, k=64, H=64, d_q=512, d_model=64, d_v=64,
         T=600),
    dict(name="k64_split_ranges_gate", dtype="bf16", qk_norm=True, memory_plus=True, n_sub=4096, k=64, H=4, d_q=512,
         d_model=256, d_v=256, T=150),
    dict(name="k64_eq_n_sub", dtype="f32", qk_norm=False, n_sub=64, k=64, H=2, d_q=128, d_model=64, d_v=64, T=40),
    dict(name="k40_f32_two_pass", dtype="f32", qk_norm=True, n_sub=2000, k=40, H=4, d_q=256, d_model=64, d_v=64, T=260),
    # any even d_query: halves stored padded with zeros to 64, 128 or 256
    dict(name="dq96_two_pass", dtype="bf16", qk_norm=True, n_sub=1100, k=32, H=4, d_q=96, d_model=64, d_v=64, T=300),
    dict(name="dq6_exhaustive", dtype="bf16", qk_norm=True, n_sub=50, k=8, H=2, d_q=6, d_model=64, d_v=64, T=64),
    dict(name="dq200_gate_eight_waves", dtype="bf16", qk_norm=True, memory_plus=True, n_sub=1030, k=16, H=32, d_q=200,
         d_model=128, d_v=128, T=1100),
    dict(name="dq258_k64", dtype="bf16", qk_norm=True, n_sub=2048, k=64, H=4, d_q=258, d_model=64, d_v=64, T=300),
    dict(name="dq2_k1", dtype="f32", qk_norm=True, n_sub=40, k=1, H=3, d_q=2, d_model=64, d_v=64, T=33),
    dict(name="dq300_f32_exhaustive", dtype="f32", qk_norm=True, n_sub=500, k=40, H=2, d_q=300, d_model=64, d_v=64,
         T=100),
    dict(name="dq62_f32_two_pass", dtype="f32", qk_norm=False, n_sub=1050, k=8, H=8, d_q=62, d_model=64, d_v=64,
         T=500),
])
def test_wide_k_and_any_even_query_width(case):
    """The boundary's full range: 1 <= k <= min(n_sub, 64) and any even d_query up to 512.
    Stage-wise and end to end against the oracle (on a spread of tokens for the large batches),
    and pkm_select from the forward's own normalised query (given in the caller's unpadded
    layout) bitwise equal to the forward's selection."""
    import sparse_key_value_amd as P
    case = dict(case)
    name = case.pop("name")
    cfg = CONFIGS["pkm_1m_bf16"].with_(name=name, memory_plus=case.pop("memory_plus", False), **case)
    say(f"boundary {cfg.name}")
    wl = _G().Workload(cfg, seed=13)
    o = run_debug(wl)
    full_check(wl, o, rows=None if cfg.T * cfg.H <= 4096 else _sample_tokens(cfg.T))
    q = _G().to_dev(o["qhat"], cfg.dtype)
    idx = torch.empty((cfg.T, cfg.H, cfg.k), dtype=torch.int32, device="cuda")
    sc = torch.empty((cfg.T, cfg.H, cfg.k), dtype=torch.float32, device="cuda")
    w = torch.empty((cfg.T, cfg.H, cfg.k), dtype=torch.float32, device="cuda")
    P.pkm_select(wl.pkm.handle, q, cfg.T, None, None, idx, sc, w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), o["idx"])
    np.testing.assert_array_equal(w.cpu().numpy(), o["w"])
    wl.close()


def test_wide_combine_rounding_tie_takes_exhaustive_path():
    """k = 34 (the combine for k > 32) with an fp32 rounding tie off the staircase.

    Half 0: sub-key 10 scores 2^25, sub-key 3 scores 2^25 - 2, every other one -1000; half 1:
    sub-key b scores 1.5 - 0.4 b / 64, all in (1.1, 1.5].  Every cell of sub-keys 10 and 3 then
    sums to 2^25 in fp32, so by flat index (a * 64 + b) the top-34 cells are (3, 0..33); the
    half-0 list is (10, 3, ...), which puts (3, 17..33) off the staircase (2 (j + 1) > 34), so
    only the exhaustive redo finds them.  The float64 oracle orders by the exact sums, (10,
    0..33); the two lists differ only inside the near-tie margin.
    """
    import sparse_key_value_amd as P
    n, dh, k = 64, 64, 34
    K = np.zeros((1, 2, n, dh), dtype=np.float32)
    K[0, 0, :, 0] = -1000.0
    K[0, 0, 10, 0], K[0, 0, 3, 0] = 2.0 ** 25, 2.0 ** 25 - 2
    K[0, 1, :, 1] = (1.5 - 0.4 * np.arange(n) / 64).astype(np.float32)
    wq = torch.zeros((64, 2 * dh), dtype=torch.float32, device="cuda")
    vals = torch.zeros((n * n, 4), dtype=torch.float32, device="cuda")
    pk = P.ProductKeyMemory(d_model=64, n_heads=1, d_query=2 * dh, n_sub=n, k=k, d_value=4, dtype="f32", qk_norm=0,
                            memory_plus=0, max_tokens=4, W_q=wq, subkeys=torch.from_numpy(K).cuda(), values=vals)
    q = np.zeros((1, 1, 2, dh), dtype=np.float32)
    q[0, 0, 0, 0] = 1.0
    q[0, 0, 1, 1] = 1.0
    hi_ = torch.empty((1, 1, 2, k), dtype=torch.int32, device="cuda")
    hs_ = torch.empty((1, 1, 2, k), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, 1, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((1, 1, k), dtype=torch.float32, device="cuda")
    w = torch.empty((1, 1, k), dtype=torch.float32, device="cuda")
    P.pkm_select(pk.handle, torch.from_numpy(q).cuda(), 1, hi_, hs_, idx, sc, w)
    torch.cuda.synchronize()
    assert hi_.cpu().numpy()[0, 0, 0, :2].tolist() == [10, 3]
    assert hi_.cpu().numpy()[0, 0, 1].tolist() == list(range(k))
    assert idx.cpu().numpy()[0, 0].tolist() == [3 * n + b for b in range(k)]
    assert (sc.cpu().numpy() == 2.0 ** 25).all()
    np.testing.assert_allclose(w.cpu().numpy(), 1.0 / k, rtol=1e-6)
    q64 = q.astype(np.float64).reshape(1, 1, 2 * dh)
    K64 = K.astype(np.float64)
    sel = O.select(q64[..., :dh], q64[..., dh:], K64[:, 0], K64[:, 1], k)
    assert sel["idx"][0, 0].tolist() == [10 * n + b for b in range(k)]
    ch = PAR.cell_choice_scores(q64[..., :dh], q64[..., dh:], K64[:, 0], K64[:, 1], idx.cpu().numpy())
    PAR.check_lists(idx.cpu().numpy(), sel["idx"], sel["score"], ch, "wide rounding-tie case")
    pk.close()


@pytest.mark.parametrize("case", [
    dict(n_sub=4096, H=4, T=700, d_q=512, k=32),      # 8-wave blocks of 32-token waves, 16M-key sub-keys
    dict(n_sub=1024, H=64, T=520, d_q=512, k=64),     # 8-wave blocks of 64-token waves, k > 32
    dict(n_sub=2048, H=4, T=150, d_q=400, k=16),      # split sub-key ranges, halves padded from 200 to 256
])
def test_fp8_bound_and_exact_bound_select_alike(case):
    """The bound pass from fp8 scores (bf16, 256-wide halves) and the exact one from bf16
    scores: both forwards match the oracle stage-wise, and they select the same lists (any
    difference would be a near-tie the rule excuses)."""
    import sparse_key_value_amd as P
    cfg = CONFIGS["pkm_1m_bf16"].with_(name=f"bounds_h{case['H']}_n{case['n_sub']}", d_model=128, d_v=128, **case)
    say(f"fp8 and exact bounds {case}")
    wl = _G().Workload(cfg, seed=17)
    rows = None if cfg.T * cfg.H <= 4096 else _sample_tokens(cfg.T)
    res = {}
    for mode in ("exact", "auto"):
        P.pkm_set_score_bound(wl.pkm.handle, mode)
        res[mode] = run_debug(wl)
        full_check(wl, res[mode], rows=rows)
    diff = res["auto"]["idx"] != res["exact"]["idx"]
    say(f"positions selected differently by the two bounds: {int(diff.sum())} of {diff.size}")
    assert diff.mean() < 1e-3
    wl.close()


def test_fp8_bound_that_overshoots_falls_back_to_exhaustive_rows():
    """Every sub-key element is 1.09375, which fp8 rounds up to 1.125: each fp8 score overstates
    the exact one by about 8, far beyond the bound's margin (about 1.7 here), so no exact
    score reaches the bound and every row holds fewer than k candidates.  Each row is then
    scored exhaustively, and the lists equal the oracle's exactly (the scores are exact in
    fp32: sums of multiples of 1/32)."""
    import sparse_key_value_amd as P
    n, dh, k, T = 256, 256, 8, 6
    K = np.full((1, 2, n, dh), 1.09375, dtype=np.float32)
    K[0, 0, :, 0] = np.arange(n) / 16.0                 # half 0: score rises with the index
    K[0, 1, :, 0] = np.arange(n)[::-1] / 16.0           # half 1: falls with the index
    kb = torch.from_numpy(K).to(torch.bfloat16).cuda()
    assert torch.equal(kb.float().cpu(), torch.from_numpy(K))       # bf16-exact
    q = np.ones((T, 1, 2, dh), dtype=np.float32)
    q[1::2, 0, 1, :] = 0.5                                           # other scales of half 1
    qb = torch.from_numpy(q).to(torch.bfloat16).cuda()
    wq = torch.zeros((64, 2 * dh), dtype=torch.bfloat16, device="cuda")
    vals = torch.zeros((n * n, 8), dtype=torch.bfloat16, device="cuda")
    pk = P.ProductKeyMemory(d_model=64, n_heads=1, d_query=2 * dh, n_sub=n, k=k, d_value=8, dtype="bf16", qk_norm=0,
                            memory_plus=0, max_tokens=T, W_q=wq, subkeys=kb, values=vals)
    q64 = q.astype(np.float64).reshape(T, 1, 2 * dh)
    sel = O.select(q64[..., :dh], q64[..., dh:], K[:, 0].astype(np.float64), K[:, 1].astype(np.float64), k)
    assert sel["half_idx"][0, 0, 0].tolist() == list(range(n - 1, n - 1 - k, -1))
    for mode in ("auto", "exact"):
        P.pkm_set_score_bound(pk.handle, mode)
        hi_ = torch.empty((T, 1, 2, k), dtype=torch.int32, device="cuda")
        hs_ = torch.empty((T, 1, 2, k), dtype=torch.float32, device="cuda")
        idx = torch.empty((T, 1, k), dtype=torch.int32, device="cuda")
        sc = torch.empty((T, 1, k), dtype=torch.float32, device="cuda")
        w = torch.empty((T, 1, k), dtype=torch.float32, device="cuda")
        P.pkm_select(pk.handle, qb, T, hi_, hs_, idx, sc, w)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(hi_.cpu().numpy(), sel["half_idx"], err_msg=mode)
        np.testing.assert_array_equal(hs_.cpu().numpy(), sel["half_score"].astype(np.float32), err_msg=mode)
        np.testing.assert_array_equal(idx.cpu().numpy(), sel["idx"], err_msg=mode)
    pk.close()


def _ord_key(x):
    """float32 -> the kernels' ordered 32-bit key (a larger float has a larger key; -0 as +0)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    b[b == 0x80000000] = 0
    return np.where((b & 0x80000000) != 0, ~b, b | np.uint32(0x80000000)).astype(np.uint32)


def _of_ord_key(o):
    o = np.asarray(o, dtype=np.uint32)
    return np.where((o & 0x80000000) != 0, o & np.uint32(0x7FFFFFFF), ~o).astype(np.uint32).view(np.float32)


@pytest.mark.parametrize("shape", [
    dict(n_sub=1100, T=600, H=64),      # 8-wave blocks, sub-keys not split: the bound in pass 1's tail
    dict(n_sub=1024, T=300, H=2),       # a small batch: split sub-key ranges, the bound from theta_kernel
])
def test_selection_bound_is_the_kth_group_maximum(shape):
    """The bound the two scoring passes select against ("Memory Layers at Scale" digest, product-key
    search: only the sub-keys that can be among a half's k best need be kept).  With the exact
    bound it is the k-th largest of the row's group maxima rounded down to the top 16 bits of its
    ordered key, so at least k sub-keys reach it, and the candidate counts are the scores at or
    above it; with the fp8 bound it is that value for fp8 scores less a margin of
    0.006 |q_c| max|K_c|.  Per (token, head, half), from the GPU's own q-hat and K-hat bytes in
    float64.  The results never depend on the bound (exact counts catch one set too high), so
    this is what pins pass 1's group maxima, their cross-lane maxima and the bit descent."""
    import sparse_key_value_amd as P
    G = _G()
    cfg = CONFIGS["pkm_1m_bf16"].with_(name="bound", d_v=64, d_model=256, memory_plus=False, **shape)
    say(f"selection bound {shape}")
    wl = G.Workload(cfg, seed=31)
    T, H, k, n, dh = wl.T, cfg.H, cfg.k, cfg.n_sub, cfg.d_h
    assert cfg.dtype == "bf16" and cfg.qk_norm and dh == 256        # the fp8 bound is built here
    gs = 0
    while -(-n // (8 << gs)) > 128:
        gs += 1
    gsz = 8 << gs
    ng = -(-n // gsz)
    assert ng >= 2 * k                                                # the two passes, not exhaustive rows
    kh = torch.empty((H, 2, n, dh), dtype=torch.bfloat16, device="cuda")
    P.pkm_copy_normalized_subkeys(wl.pkm.handle, kh)
    K = O.to_f64(G.to_host(kh), "bf16")
    got = {}
    for mode in ("exact", "auto"):
        P.pkm_set_score_bound(wl.pkm.handle, mode)
        qh = torch.empty((T, H, 2, dh), dtype=torch.bfloat16, device="cuda")
        th = torch.empty((T, H, 2), dtype=torch.float32, device="cuda")
        ct = torch.empty((T, H, 2, 2), dtype=torch.int32, device="cuda")
        out = torch.empty((T, cfg.d_out), dtype=torch.bfloat16, device="cuda")
        P.pkm_forward_debug(wl.pkm.handle, wl.dev["x"], T, out, {"qhat": qh, "theta": th, "counts": ct})
        torch.cuda.synchronize()
        got[mode] = (G.to_host(qh), th.cpu().numpy(), ct.cpu().numpy())
    assert np.array_equal(got["exact"][0], got["auto"][0])
    Q = O.to_f64(got["exact"][0], "bf16")
    th_x, ct_x = got["exact"][1], got["exact"][2]
    th_8 = got["auto"][1]
    n_near = n_rewritten = 0
    far = []
    for h in range(H):
        for c in range(2):
            s = Q[:, h, c] @ K[h, c].T                                    # [T, n] exact scores
            gm = np.full((T, ng * gsz), -np.inf)
            gm[:, :n] = s
            gm = gm.reshape(T, ng, gsz).max(axis=2)
            kth = -np.sort(-gm, axis=1)[:, k - 1]
            tol = 1e-3 * np.maximum(1.0, np.abs(kth))                     # fp32 sums against float64
            window = np.abs(kth) * 2.0 ** -7 + tol                        # rounded down to 16 bits
            t = th_x[:, h, c].astype(np.float64)
            assert np.all(t <= kth + tol) and np.all(t >= kth - window), (h, c)
            # the GPU's bound is the float64 k-th group maximum, truncated, up to the fp32 sums
            want = _of_ord_key(_ord_key(kth.astype(np.float32)) & np.uint32(0xFFFF0000)).astype(np.float64)
            assert np.mean(np.abs(t - want) <= tol) > 0.99, (h, c)
            cnt = (s >= t[:, None]).sum(axis=1)
            near = (np.abs(s - t[:, None]) <= tol[:, None]).sum(axis=1)
            c0, c1 = ct_x[:, h, c, 0], ct_x[:, h, c, 1]
            rewritten = (c0 == k) & (c1 == 0) & (cnt != k)                # rows the overflow pass redid
            ok = rewritten | (np.abs(c0 + c1 - cnt) <= near)
            assert ok.all() and np.all((c0 + c1)[~rewritten] >= k), (h, c)
            n_near += int((near > 0).sum())
            n_rewritten += int(rewritten.sum())
            # the fp8 estimate: near the k-th maximum less the margin
            margin = 0.006 * np.linalg.norm(Q[:, h, c], axis=1) * np.linalg.norm(K[h, c], axis=1).max()
            dev = np.abs(th_8[:, h, c] - (kth - margin))
            assert np.all(dev <= 2 * margin + window), (h, c, float(dev.max()), float(margin.max()))
            far.append(np.mean(dev > margin))
    say(f"  rows with a score within the fp32 tolerance of the bound: {n_near}; rewritten rows: {n_rewritten}; "
        f"fp8 bound off by more than its margin: {max(far):.3%} of rows at worst")
    assert max(far) < 0.05


@pytest.mark.parametrize("shape", [
    dict(n_sub=256, T=300),             # few sub-keys: every row scored exhaustively
    dict(n_sub=1100, T=600, H=64),      # the two MFMA passes in 8-wave blocks, theta, overflow scan
    dict(n_sub=1100, T=200),            # a small batch: split sub-key ranges, atomic candidate counts
])
def test_forward_in_a_hip_graph(shape):
    """The forward allocates nothing and never waits on the host, so it can be captured in a
    HIP graph: every replay equals the eager forward bitwise, also after the captured input
    changes, with eager forwards and other work between the replays."""
    import sparse_key_value_amd as P
    G = _G()
    cfg = CONFIGS["pkm_1m_bf16"].with_(name="graph", d_v=256, d_model=256, memory_plus=True, **shape)
    say(f"forward in a HIP graph {shape}")
    wl = G.Workload(cfg, seed=21)
    T, H, k = wl.T, cfg.H, cfg.k
    x = wl.dev["x"].clone()
    x_other = G.to_dev(S.make_inputs(cfg, 22, T=T)["x"], cfg.dtype)

    def buffers():
        return (torch.empty((T, cfg.d_out), dtype=torch.bfloat16, device="cuda"),
                torch.empty((T, H, k), dtype=torch.int32, device="cuda"),
                torch.empty((T, H, k), dtype=torch.float32, device="cuda"))

    def eager(inp):
        o, i, w = buffers()
        P.pkm_forward(wl.pkm.handle, inp, T, o, i, w)
        torch.cuda.synchronize()
        return [t.view(torch.int16) if t.dtype == torch.bfloat16 else t for t in (o, i, w)]

    ref = eager(x)          # also creates every GEMM plan before the capture
    ref_other = eager(x_other)
    og, ig, wg = buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        P.pkm_forward(wl.pkm.handle, x, T, og, ig, wg)
    for rep in range(3):
        src = x_other if rep == 1 else wl.dev["x"]
        x.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = ref_other if rep == 1 else ref
        for a, b in zip((og.view(torch.int16), ig, wg), want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager forward"
        eager(x_other)       # eager work on the same handle between replays
        torch.randn(1 << 20, device="cuda").sum().item()
    wl.close()
