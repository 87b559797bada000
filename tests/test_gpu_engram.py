"""GPU parity of the hashed n-gram lookup (Engram review: multi-head hashing, key
equation 1; context-aware gate, key equation 2) against the oracle, through the C ABI.

Table rows are integer results: compared bitwise for every token.  The embedding e
(an fp32 sum of stored values) is held to 1e-4 of each row's largest magnitude, the
gate to 1e-5, and the output to the per-dtype bar (1e-4 fp32, 2e-2 bf16, per row)
plus, for bf16, one bf16 ulp of the float64 result.
"""

from __future__ import annotations

import gc
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle import engram as E  # noqa: E402
from synth import configs as C  # noqa: E402
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


def _to_dev(a, dtype):
    from tests.gpu_util import to_dev
    return to_dev(a, dtype)


def _to_host(t):
    from tests.gpu_util import to_host
    return t if isinstance(t, np.ndarray) else to_host(t)


class Lookup:
    """One Engram workload on the GPU: ids, hidden states, multipliers, tables."""

    def __init__(self, cfg, seed=0, T=None, ids=None, tables=None):
        import sparse_key_value_amd as P
        from synth import device as SD
        from tests.gpu_util import TORCH_DT

        self.P, self.cfg, self.seed = P, cfg, seed
        inp = S.make_engram_inputs(cfg, seed, T=T)
        if ids is not None:
            inp["ids"] = np.asarray(ids, dtype=np.int32)
            inp["h"] = np.ascontiguousarray(S.hidden_states(seed, len(ids), cfg.d, cfg.dtype))
        self.inp, self.T = inp, len(inp["ids"])
        self.ids = torch.from_numpy(inp["ids"]).cuda()
        self.h = _to_dev(inp["h"], cfg.dtype)
        self.mult = torch.from_numpy(inp["mult"].view(np.int64)).cuda()
        self.compress = torch.from_numpy(inp["compress"]).cuda() if inp["compress"] is not None else None
        if tables is None:
            tables = torch.empty((cfg.total_rows, cfg.head_dim), dtype=TORCH_DT[cfg.dtype], device="cuda")
            SD.fill_values(tables, seed, tid=S.TID_ENGRAM)
        self.tables = tables
        self.ecfg = P.make_engram_config(cfg.min_order, cfg.n_orders, cfg.heads, cfg.head_dim, cfg.table_rows,
                                         cfg.vocab, cfg.dtype, cfg.residual, cfg.norm_eps)

    def rows(self):
        r = torch.full((self.T, self.cfg.heads, self.cfg.n_orders), -1, dtype=torch.int32, device="cuda")
        self.P.engram_hash(self.ecfg, self.ids, self.T, self.cfg.seq_len, self.compress, self.mult, r)
        torch.cuda.synchronize()
        return r.cpu().numpy()

    def forward(self):
        from tests.gpu_util import TORCH_DT
        out = torch.empty((self.T, self.cfg.d), dtype=TORCH_DT[self.cfg.dtype], device="cuda")
        e = torch.full((self.T, self.cfg.d), float("nan"), dtype=torch.float32, device="cuda")
        a = torch.full((self.T,), float("nan"), dtype=torch.float32, device="cuda")
        self.P.engram_forward(self.ecfg, self.tables, self.ids, self.T, self.cfg.seq_len, self.compress, self.mult,
                              self.h, out, e, a)
        torch.cuda.synchronize()
        return _to_host(out), e.cpu().numpy(), a.cpu().numpy()

    def rows_of(self, r):
        return E.to_f64(S.engram_table_rows(self.seed, r, self.cfg.head_dim, self.cfg.dtype), self.cfg.dtype)

    def oracle(self, tokens=None):
        """Oracle on all tokens, or on `tokens` (each with its full n-gram context)."""
        cfg, inp = self.cfg, self.inp
        rows = E.hash_rows(inp["ids"], cfg.seq_len, inp["mult"], cfg.table_rows, cfg.min_order, cfg.vocab,
                           inp["compress"])
        sel = np.arange(self.T) if tokens is None else np.asarray(tokens)
        e = E.lookup(self.rows_of, rows[sel], cfg.head_dim)
        h = E.to_f64(inp["h"][sel], cfg.dtype)
        alpha = E.gate(h, e, cfg.norm_eps)
        out = alpha[:, None] * e + (h if cfg.residual else 0.0)
        return rows, e, alpha, out


def _check(L, tokens=None):
    cfg = L.cfg
    rows_gpu = L.rows()
    out, e, a = L.forward()
    rows, e_ref, a_ref, out_ref = L.oracle(tokens)
    np.testing.assert_array_equal(rows_gpu, rows, err_msg="engram_hash rows")
    sel = np.arange(L.T) if tokens is None else np.asarray(tokens)
    PAR.check_rows(e[sel], e_ref, 1e-4, "e")
    np.testing.assert_allclose(a[sel], a_ref, rtol=0, atol=1e-5, err_msg="alpha")
    got = E.to_f64(out[sel], cfg.dtype) if cfg.dtype == "bf16" else out[sel].astype(np.float64)
    PAR.check_rows(got, out_ref, PAR.TOL[cfg.dtype], "out")
    if cfg.dtype == "bf16":
        PAR.check_bf16_rounded(out[sel], out_ref, 1e-5, "out")
    return rows_gpu


@pytest.mark.parametrize("name", ["engram_tiny_f32", "engram_compress_bf16"])
def test_engram_small_workloads_every_token(name):
    cfg = C.ENGRAM_CONFIGS[name]
    say(f"engram {name} T={cfg.T}")
    _check(Lookup(cfg, seed=3))


@pytest.mark.parametrize("shape", [
    dict(T=1, seq_len=1), dict(T=5, seq_len=3), dict(T=131, seq_len=7),
    dict(min_order=1, n_orders=4, T=97, seq_len=50),          # orders 1..4
    dict(min_order=5, n_orders=4, T=64, seq_len=64),          # orders 5..8, the longest
    dict(heads=1, head_dim=8, T=40, seq_len=40),              # one 16-byte slice per token... in f32: 2
    dict(heads=16, head_dim=128, dtype="bf16", T=70, seq_len=70),  # 4096-byte tokens, four slices per lane
    dict(heads=3, head_dim=24, dtype="bf16", T=50, seq_len=10, residual=True),  # slices not a multiple of 64
    # 64 heads x 4 orders: 256 (order, head) pairs, four per lane
    dict(heads=64, head_dim=8, min_order=1, n_orders=4, T=50, seq_len=20),
    dict(heads=64, head_dim=32, dtype="bf16", min_order=2, n_orders=4, T=45, seq_len=45),  # and 4096-byte tokens
])
def test_engram_edge_shapes(shape):
    cfg = C.ENGRAM_CONFIGS["engram_tiny_f32"].with_(**shape)
    say(f"engram edge {shape}")
    _check(Lookup(cfg, seed=5))


def test_engram_out_of_range_ids_read_as_zero():
    cfg = C.ENGRAM_CONFIGS["engram_compress_bf16"].with_(T=12, seq_len=6)
    ids = [3, -1, 4999, 5000, 7, 1 << 30, -(1 << 31), 2, 2, 0, 5001, 9]
    L = Lookup(cfg, seed=1, ids=ids)
    rows = _check(L)
    # ids -1, 5000, 2^30, -2^31 and 5001 hash like id 0
    zero = Lookup(cfg, seed=1, ids=[3, 0, 4999, 0, 7, 0, 0, 2, 2, 0, 0, 9]).rows()
    np.testing.assert_array_equal(rows, zero)


def test_engram_deterministic_and_hash_matches_forward_rows():
    cfg = C.ENGRAM_CONFIGS["engram_compress_bf16"]
    L = Lookup(cfg, seed=2)
    a = L.forward()
    b = L.forward()
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x.view(np.uint8), y.view(np.uint8))


def test_engram_zero_tokens_is_a_no_op():
    cfg = C.ENGRAM_CONFIGS["engram_tiny_f32"]
    L = Lookup(cfg, seed=0, T=4)
    L.P.engram_forward(L.ecfg, L.tables, L.ids, 0, cfg.seq_len, None, L.mult, L.h, L.h, None, None)
    L.P.engram_hash(L.ecfg, L.ids, 0, cfg.seq_len, None, L.mult, L.ids)
    torch.cuda.synchronize()


def test_engram_full_size_as_benchmarked():
    """16,384 Zipf token ids, 2- and 3-grams x 8 heads into 16 tables of 2,097,143 rows x
    128 bf16 (8 GiB): rows bitwise for every token, values on 96 sampled tokens."""
    cfg = C.ENGRAM_CONFIGS[C.ENGRAM_HEADLINE]
    say(f"engram full size {cfg.name}: filling {cfg.total_rows * cfg.head_dim * 2 / 2**30:.1f} GiB")
    L = Lookup(cfg, seed=0)
    rng = np.random.default_rng(7)
    tokens = np.unique(np.concatenate([[0, 1, 2, cfg.T - 1], rng.choice(cfg.T, 92, replace=False)]))
    rows = _check(L, tokens)
    # properties on every token: each row inside its own table
    o = np.arange(cfg.n_orders)[None, None, :]
    k = np.arange(cfg.heads)[None, :, None]
    base = (o * cfg.heads + k) * cfg.table_rows
    assert np.all(rows >= base) and np.all(rows < base + cfg.table_rows)
    out, e, a = L.forward()
    assert np.all((a > 0) & (a < 1)) and np.isfinite(e).all()
    del L


def _staged(L, tables):
    from tests.gpu_util import TORCH_DT
    cfg = L.cfg
    st = torch.full((L.T, cfg.n_orders, cfg.d), float("nan"), dtype=TORCH_DT[cfg.dtype], device="cuda")
    L.P.engram_prefetch(L.ecfg, tables, L.ids, L.T, cfg.seq_len, L.compress, L.mult, st)
    out = torch.empty((L.T, cfg.d), dtype=TORCH_DT[cfg.dtype], device="cuda")
    e = torch.empty((L.T, cfg.d), dtype=torch.float32, device="cuda")
    a = torch.empty((L.T,), dtype=torch.float32, device="cuda")
    L.P.engram_forward_staged(L.ecfg, st, L.h, L.T, out, e, a)
    torch.cuda.synchronize()
    return _to_host(st), _to_host(out), e.cpu().numpy(), a.cpu().numpy()


def _check_staged(L, staged, out, e, a):
    """Staged rows are the oracle's table rows bitwise; the staged lookup equals the direct one bitwise."""
    cfg = L.cfg
    rows = E.hash_rows(L.inp["ids"], cfg.seq_len, L.inp["mult"], cfg.table_rows, cfg.min_order, cfg.vocab,
                       L.inp["compress"])                                      # [T, heads, orders]
    want = S.engram_table_rows(L.seed, rows.transpose(0, 2, 1).reshape(-1), cfg.head_dim, cfg.dtype)
    np.testing.assert_array_equal(np.asarray(staged).reshape(L.T, cfg.n_orders, cfg.heads, cfg.head_dim),
                                  want.reshape(L.T, cfg.n_orders, cfg.heads, cfg.head_dim), err_msg="staged rows")
    o2, e2, a2 = L.forward()
    for x, y, n in ((out, o2, "out"), (e, e2, "e"), (a, a2, "alpha")):
        np.testing.assert_array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8), err_msg=n)


@pytest.mark.parametrize("name", ["engram_tiny_f32", "engram_compress_bf16"])
def test_engram_prefetch_from_device_tables(name):
    cfg = C.ENGRAM_CONFIGS[name]
    say(f"engram prefetch (device tables) {name}")
    L = Lookup(cfg, seed=3)
    _check_staged(L, *_staged(L, L.tables))


@pytest.mark.parametrize("name", ["engram_compress_bf16", "engram_zipf_2m_bf16"])
def test_engram_prefetch_from_pinned_host_tables(name):
    """Tables in pinned host memory, read by the kernel over the host link."""
    cfg = C.ENGRAM_CONFIGS[name]
    say(f"engram prefetch (pinned host tables) {name}")
    L = Lookup(cfg, seed=0)
    host = torch.empty(L.tables.shape, dtype=L.tables.dtype, pin_memory=True)
    host.copy_(L.tables)
    torch.cuda.synchronize()
    dev = L.tables
    L.tables = None
    del dev
    torch.cuda.empty_cache()
    staged, out, e, a = _staged(L, host)
    L.tables = host.cuda()
    _check_staged(L, staged, out, e, a)


def test_engram_prefetch_refuses_pageable_host_memory():
    import sparse_key_value_amd as P
    cfg = C.ENGRAM_CONFIGS["engram_tiny_f32"]
    L = Lookup(cfg, seed=1, T=8)
    pageable = torch.empty(L.tables.shape, dtype=L.tables.dtype)          # plain host memory
    st = torch.empty((L.T, cfg.n_orders, cfg.d), dtype=torch.float32, device="cuda")
    with pytest.raises(P.PkmError) as ex:
        P.engram_prefetch(L.ecfg, pageable, L.ids, L.T, cfg.seq_len, None, L.mult, st)
    assert ex.value.code == P.PKM_EINVAL and "pinned" in str(ex.value)


def test_lookup_in_a_hip_graph():
    """engram_forward allocates nothing and never waits on the host: captured in a HIP graph,
    every replay equals the eager lookup bitwise, also after the captured ids change."""
    from tests.gpu_util import TORCH_DT
    cfg = C.ENGRAM_CONFIGS["engram_compress_bf16"]
    say("engram lookup in a HIP graph")
    L = Lookup(cfg, seed=5)
    ids0 = L.ids.clone()
    ids1 = torch.from_numpy(S.make_engram_inputs(cfg, 6)["ids"][:L.T].copy()).cuda()

    def run(out, e, a):
        L.P.engram_forward(L.ecfg, L.tables, L.ids, L.T, cfg.seq_len, L.compress, L.mult, L.h, out, e, a)

    def bufs():
        return (torch.empty((L.T, cfg.d), dtype=TORCH_DT[cfg.dtype], device="cuda"),
                torch.empty((L.T, cfg.d), dtype=torch.float32, device="cuda"),
                torch.empty((L.T,), dtype=torch.float32, device="cuda"))

    want = {}
    for name, ids in (("0", ids0), ("1", ids1)):
        L.ids.copy_(ids)
        b = bufs()
        run(*b)
        torch.cuda.synchronize()
        want[name] = [t.clone() for t in b]
    g_bufs = bufs()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(*g_bufs)
    for rep, name in enumerate(("0", "1", "0")):
        L.ids.copy_(ids0 if name == "0" else ids1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(g_bufs, want[name]):
            assert torch.equal(a, b), f"replay {rep} differs from the eager lookup"
        run(*bufs())
        torch.cuda.synchronize()
