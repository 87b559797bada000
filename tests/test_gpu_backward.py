"""GPU parity of the EmbeddingBag backward and the sparse update, through the C ABI.

Integer results (the distinct rows, their count) are compared exactly; dw, ds and the
row gradients (fp32 sums of fp32 products) to 1e-4 of each row's largest magnitude
against the float64 oracle; the updated table stage-wise (the oracle applies the GPU's
own gradient) to one storage ulp, with every untouched row bitwise unchanged.
"""

from __future__ import annotations

import gc
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle import backward as B  # noqa: E402
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


def _run(table, n_rows, dim, dt, idx, w, dy, group, update=False, lr=0.0, want_grad=True, grad_to_host=True):
    import sparse_key_value_amd as P
    n_bags, bag = idx.shape
    n = n_bags * bag
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    idx_d, w_d, dy_d = dev(idx.astype(np.int32)), dev(w.astype(np.float32)), dev(dy.astype(np.float32))
    dw = torch.full((n_bags, bag), float("nan"), device="cuda")
    ds = torch.full((n_bags, bag), float("nan"), device="cuda")
    rows = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    grad = torch.full((n, dim), float("nan"), device="cuda") if want_grad else None
    nu = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    ws_bytes = P.pkm_bag_backward_workspace_size(n_bags, bag, n_rows)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    P.pkm_bag_backward(table, n_rows, dim, dt, idx_d, w_d, dy_d, n_bags, bag, dw=dw, ds=ds, softmax_group=group,
                       rows=rows, grad=grad, n_unique=nu, update=update, lr=lr, workspace=ws)
    torch.cuda.synchronize()
    U = int(nu.item())
    g = None
    if want_grad:
        g = grad[:U].cpu().numpy() if grad_to_host else grad[:U]
    return {"dw": dw.cpu().numpy(), "ds": ds.cpu().numpy(), "U": U, "rows": rows[:U].cpu().numpy(), "grad": g}


def _check(got, table_rows_of, n_rows, idx, w, dy, group, tokens=None):
    sel = np.arange(idx.shape[0]) if tokens is None else np.asarray(tokens)
    dw_ref = B.grad_weights(table_rows_of, idx[sel], dy[sel], n_rows)
    PAR.check_rows(got["dw"][sel], dw_ref, 1e-4, "dw")
    ds_ref = B.softmax_backward(w[sel].astype(np.float64), got["dw"][sel].astype(np.float64), group)
    np.testing.assert_allclose(got["ds"][sel], ds_ref, rtol=1e-5, atol=1e-6 * np.abs(ds_ref).max())
    if tokens is None:
        rows_ref, grad_ref = B.grad_rows(idx, w, dy, n_rows)
        np.testing.assert_array_equal(got["rows"], rows_ref)
        assert got["U"] == len(rows_ref)
        if got["grad"] is not None:
            PAR.check_rows(got["grad"], grad_ref, 1e-4, "row gradients")


def _one_ulp(got_stored, ref64, dt):
    g = O.to_f64(got_stored, dt)
    mag = np.maximum(np.abs(ref64), 1e-30)
    ulp = 2.0 ** (np.floor(np.log2(mag)) - (7 if dt == "bf16" else 23))
    assert np.all(np.abs(g - ref64) <= ulp), f"update beyond one ulp: {np.abs(g - ref64).max():.3e}"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_small_with_duplicates_and_out_of_range(dt):
    from tests.gpu_util import TORCH_DT, to_dev, to_host
    rng = np.random.default_rng(0)
    n_rows, dim, n_bags, k, H = 400, 64, 120, 8, 2
    bag = H * k
    idx = rng.integers(-3, n_rows + 3, size=(n_bags, bag))          # some out of range
    idx[:5, :4] = 17                                               # a row many times, also within a bag
    s = rng.standard_normal((n_bags, H, k))
    w = np.exp(s - s.max(-1, keepdims=True))
    w = (w / w.sum(-1, keepdims=True)).reshape(n_bags, bag).astype(np.float32)
    dy = rng.standard_normal((n_bags, dim)).astype(np.float32)
    host = S.value_rows(9, np.arange(n_rows), dim, dt)
    table = to_dev(host, dt)
    say(f"bag backward small {dt}")
    got = _run(table, n_rows, dim, dt, idx, w, dy, k)
    rows_of = lambda r: O.to_f64(host[np.asarray(r)], dt)
    _check(got, rows_of, n_rows, idx, w.astype(np.float64), dy.astype(np.float64), k)
    # the update, stage-wise from the GPU's gradient; untouched rows unchanged
    before = to_host(table).copy()
    lr = 0.125
    got2 = _run(table, n_rows, dim, dt, idx, w, dy, k, update=True, lr=lr)
    after = to_host(table)
    np.testing.assert_array_equal(got2["rows"], got["rows"])
    # with the update, dw and ds come from the rows the update reads: still the old rows
    _check(got2, rows_of, n_rows, idx, w.astype(np.float64), dy.astype(np.float64), k)
    ref = O.to_f64(before[got["rows"]], dt) - lr * got2["grad"].astype(np.float64)
    _one_ulp(after[got["rows"]], ref, dt)
    untouched = np.setdiff1d(np.arange(n_rows), got["rows"])
    np.testing.assert_array_equal(np.asarray(after[untouched]).view(np.uint8),
                                  np.asarray(before[untouched]).view(np.uint8))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_update_alone_matches_update_with_outputs(dt):
    """The update with no other output asked for (no sort outputs, no gradient) leaves the
    same table, bit for bit, as the update that also writes the gradients, and that table
    is one storage ulp from the stage-wise oracle; rows repeated within and across bags."""
    import sparse_key_value_amd as P
    from tests.gpu_util import to_dev, to_host
    rng = np.random.default_rng(7)
    n_rows, dim, n_bags, bag = 300, 96 if dt == "bf16" else 64, 200, 24
    idx = rng.integers(-2, n_rows + 2, size=(n_bags, bag))
    idx[:9, :6] = 5                                                # one row 54 times
    idx[20, 3] = idx[20, 11] = 299                                 # a row twice in one bag, last row
    w = rng.random((n_bags, bag)).astype(np.float32)
    dy = rng.standard_normal((n_bags, dim)).astype(np.float32)
    host = S.value_rows(11, np.arange(n_rows), dim, dt)
    t1, t2 = to_dev(host, dt), to_dev(host, dt)
    lr = 0.25
    say(f"bag update alone {dt}")
    ref = _run(t1, n_rows, dim, dt, idx, w, dy, 8, update=True, lr=lr)
    ws = torch.empty(P.pkm_bag_backward_workspace_size(n_bags, bag, n_rows), dtype=torch.uint8, device="cuda")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    P.pkm_bag_backward(t2, n_rows, dim, dt, dev(idx.astype(np.int32)), dev(w), dev(dy), n_bags, bag, update=True,
                       lr=lr, workspace=ws)
    torch.cuda.synchronize()
    # ds alone with the update: dw goes to the workspace
    t3 = to_dev(host, dt)
    ds3 = torch.full((n_bags, bag), float("nan"), device="cuda")
    P.pkm_bag_backward(t3, n_rows, dim, dt, dev(idx.astype(np.int32)), dev(w), dev(dy), n_bags, bag, ds=ds3,
                       softmax_group=8, update=True, lr=lr, workspace=ws)
    torch.cuda.synchronize()
    a1, a2 = to_host(t1), to_host(t2)
    np.testing.assert_array_equal(np.asarray(a2).view(np.uint8), np.asarray(a1).view(np.uint8))
    np.testing.assert_array_equal(np.asarray(to_host(t3)).view(np.uint8), np.asarray(a1).view(np.uint8))
    np.testing.assert_array_equal(ds3.cpu().numpy(), ref["ds"])
    rows_ref, grad_ref = B.grad_rows(idx, w.astype(np.float64), dy.astype(np.float64), n_rows)
    np.testing.assert_array_equal(ref["rows"], rows_ref)
    PAR.check_rows(ref["grad"], grad_ref, 1e-4, "row gradients")
    _one_ulp(a2[rows_ref], O.to_f64(host[rows_ref], dt) - lr * ref["grad"].astype(np.float64), dt)
    untouched = np.setdiff1d(np.arange(n_rows), rows_ref)
    np.testing.assert_array_equal(np.asarray(a2[untouched]).view(np.uint8), np.asarray(host[untouched]).view(np.uint8))


@pytest.mark.parametrize("dt,dim", [("bf16", 64), ("f32", 96), ("bf16", 1024), ("bf16", 1280), ("f32", 1536),
                                    ("f32", 2048), ("bf16", 2048)])
def test_fused_step_shapes(dt, dim):
    """dw, ds, gradients and the update in one call, for widths that give one, two and
    four waves per token and one or two 16-byte slices per lane (some lanes idle)."""
    from tests.gpu_util import to_dev, to_host
    rng = np.random.default_rng(dim)
    n_rows, n_bags, k, H = 700, 64, 8, 4
    bag = H * k
    idx = rng.integers(-1, n_rows + 1, size=(n_bags, bag))
    idx[:6, :5] = 3                                                # a shared row, also within bags
    idx[40, 7] = idx[41, 7] = n_rows - 1
    s_ = rng.standard_normal((n_bags, H, k))
    w = np.exp(s_ - s_.max(-1, keepdims=True))
    w = (w / w.sum(-1, keepdims=True)).reshape(n_bags, bag).astype(np.float32)
    dy = rng.standard_normal((n_bags, dim)).astype(np.float32)
    host = S.value_rows(13, np.arange(n_rows), dim, dt)
    table = to_dev(host, dt)
    lr = 0.5
    say(f"bag fused step {dt} dim {dim}")
    got = _run(table, n_rows, dim, dt, idx, w, dy, k, update=True, lr=lr)
    rows_of = lambda r: O.to_f64(host[np.asarray(r)], dt)
    _check(got, rows_of, n_rows, idx, w.astype(np.float64), dy.astype(np.float64), k)
    after = to_host(table)
    _one_ulp(after[got["rows"]], O.to_f64(host[got["rows"]], dt) - lr * got["grad"].astype(np.float64), dt)
    untouched = np.setdiff1d(np.arange(n_rows), got["rows"])
    np.testing.assert_array_equal(np.asarray(after[untouched]).view(np.uint8),
                                  np.asarray(host[untouched]).view(np.uint8))


@pytest.mark.parametrize("dt,dim,n_bags,H,k", [("bf16", 2048, 3, 2, 5), ("f32", 96, 5, 2, 5), ("f32", 1536, 4, 3, 3),
                                             ("bf16", 64, 1, 1, 1)])
def test_fused_step_ragged_bags(dt, dim, n_bags, H, k):
    """Bags whose length is not a multiple of the update kernel's batch of rows in flight
    (8, or 4 with two slices per lane): 10, 9 and 1 entries; one bag alone."""
    from tests.gpu_util import to_dev, to_host
    rng = np.random.default_rng(dim + 7 * H + k)
    n_rows = 40
    bag = H * k
    idx = rng.integers(-1, n_rows + 1, size=(n_bags, bag))
    idx[0, 0] = idx[-1, -1] = 7                                     # a shared row across bags (or a lone entry)
    s_ = rng.standard_normal((n_bags, H, k))
    w = np.exp(s_ - s_.max(-1, keepdims=True))
    w = (w / w.sum(-1, keepdims=True)).reshape(n_bags, bag).astype(np.float32)
    dy = rng.standard_normal((n_bags, dim)).astype(np.float32)
    host = S.value_rows(17, np.arange(n_rows), dim, dt)
    table = to_dev(host, dt)
    lr = 0.5
    say(f"bag fused step ragged {dt} dim {dim} bags {n_bags}x{bag}")
    got = _run(table, n_rows, dim, dt, idx, w, dy, k, update=True, lr=lr)
    rows_of = lambda r: O.to_f64(host[np.asarray(r)], dt)
    _check(got, rows_of, n_rows, idx, w.astype(np.float64), dy.astype(np.float64), k)
    after = to_host(table)
    _one_ulp(after[got["rows"]], O.to_f64(host[got["rows"]], dt) - lr * got["grad"].astype(np.float64), dt)
    untouched = np.setdiff1d(np.arange(n_rows), got["rows"])
    np.testing.assert_array_equal(np.asarray(after[untouched]).view(np.uint8),
                                  np.asarray(host[untouched]).view(np.uint8))


@pytest.mark.parametrize("dt,dim,n_rows", [("bf16", 256, 40), ("f32", 64, 5000)])
def test_largest_bags(dt, dim, n_rows):
    """Bags of 2,048 entries (64 heads x k = 32, the largest bag the backward takes): dw, ds,
    the per-row gradients and the update, over 40 rows (every row shared by about 150
    entries of three bags) and over 5,000 rows."""
    from tests.gpu_util import to_dev, to_host
    rng = np.random.default_rng(dim + n_rows)
    n_bags, H, k = 3, 64, 32
    bag = H * k
    idx = rng.integers(-1, n_rows + 1, size=(n_bags, bag))
    s_ = rng.standard_normal((n_bags, H, k))
    w = np.exp(s_ - s_.max(-1, keepdims=True))
    w = (w / w.sum(-1, keepdims=True)).reshape(n_bags, bag).astype(np.float32)
    dy = rng.standard_normal((n_bags, dim)).astype(np.float32)
    host = S.value_rows(19, np.arange(n_rows), dim, dt)
    table = to_dev(host, dt)
    lr = 0.25
    say(f"bag fused step, largest bags {dt} dim {dim} rows {n_rows}")
    got = _run(table, n_rows, dim, dt, idx, w, dy, k, update=True, lr=lr)
    rows_of = lambda r: O.to_f64(host[np.asarray(r)], dt)
    _check(got, rows_of, n_rows, idx, w.astype(np.float64), dy.astype(np.float64), k)
    after = to_host(table)
    _one_ulp(after[got["rows"]], O.to_f64(host[got["rows"]], dt) - lr * got["grad"].astype(np.float64), dt)
    untouched = np.setdiff1d(np.arange(n_rows), got["rows"])
    np.testing.assert_array_equal(np.asarray(after[untouched]).view(np.uint8),
                                  np.asarray(host[untouched]).view(np.uint8))


def test_deterministic():
    from tests.gpu_util import to_dev
    rng = np.random.default_rng(1)
    n_rows, dim, n_bags, bag = 50, 128, 400, 32                   # heavy reuse: ~256 entries per row
    idx = rng.integers(0, n_rows, size=(n_bags, bag))
    w = rng.random((n_bags, bag)).astype(np.float32)
    dy = rng.standard_normal((n_bags, dim)).astype(np.float32)
    table = to_dev(S.value_rows(2, np.arange(n_rows), dim, "bf16"), "bf16")
    a = _run(table, n_rows, dim, "bf16", idx, w, dy, 8)
    b = _run(table, n_rows, dim, "bf16", idx, w, dy, 8)
    for k in ("dw", "ds", "rows", "grad"):
        np.testing.assert_array_equal(np.asarray(a[k]).view(np.uint8), np.asarray(b[k]).view(np.uint8))


def test_forward_indices_pkm_1m():
    """The backward of a real forward's gather (1M-key table, 4 heads x k = 32)."""
    from tests import gpu_util as G
    cfg = CONFIGS["pkm_1m_bf16"]
    T = 256
    wl = G.Workload(cfg, seed=0, T=T)
    o = wl.forward_debug()
    idx = o["idx"].cpu().numpy().reshape(T, cfg.H * cfg.k)
    w = o["w"].cpu().numpy().reshape(T, cfg.H * cfg.k)
    dy = np.random.default_rng(3).standard_normal((T, cfg.d_v)).astype(np.float32)
    say("bag backward on pkm_1m forward indices")
    got = _run(wl.values, cfg.N, cfg.d_v, cfg.dtype, idx, w, dy, cfg.k)
    _check(got, lambda r: O.to_f64(wl.host_rows(r), cfg.dtype), cfg.N, idx, w.astype(np.float64),
           dy.astype(np.float64), cfg.k)
    wl.close()


def test_full_size_sampled():
    """16,384 tokens x 128 entries over the 16M-key, 64 GiB table, as benchmarked: the
    distinct rows exactly, dw/ds on sampled tokens, gradients of sampled rows."""
    from tests import gpu_util as G
    cfg = CONFIGS["memplus_16m_bf16"]
    T = cfg.T
    wl = G.Workload(cfg, seed=0, T=T)
    o = wl.forward_debug()
    bag = cfg.H * cfg.k
    idx = o["idx"].cpu().numpy().reshape(T, bag)
    w = o["w"].cpu().numpy().reshape(T, bag)
    del o
    dy = np.random.default_rng(4).standard_normal((T, cfg.d_v)).astype(np.float32)
    say("bag backward full size")
    got = _run(wl.values, cfg.N, cfg.d_v, cfg.dtype, idx, w, dy, cfg.k, grad_to_host=False)
    rng = np.random.default_rng(5)
    tokens = np.sort(rng.choice(T, 24, replace=False))
    rows_of = lambda r: O.to_f64(wl.host_rows(r), cfg.dtype)
    _check(got, rows_of, cfg.N, idx, w.astype(np.float64), dy.astype(np.float64), cfg.k, tokens=tokens)
    uniq = np.unique(idx)
    np.testing.assert_array_equal(got["rows"], uniq)
    # sampled rows: the most repeated ones and random ones
    vals, counts = np.unique(idx, return_counts=True)
    pick = np.concatenate([vals[np.argsort(-counts)[:8]], rng.choice(vals, 24, replace=False)])
    flat_i, flat_w = idx.reshape(-1), w.reshape(-1).astype(np.float64)
    for r in pick:
        pos = np.nonzero(flat_i == r)[0]
        ref = np.sum(flat_w[pos, None] * dy[pos // bag].astype(np.float64), axis=0)
        u = int(np.searchsorted(got["rows"], r))
        PAR.check_rows(got["grad"][u].cpu().numpy()[None], ref[None], 1e-4, f"gradient of row {r}")
    del got
    # the update alone, as benchmarked (distinct rows and their count, no gradients): sampled
    # touched rows against the float64 oracle's step, sampled untouched rows unchanged
    import sparse_key_value_amd as P
    from tests.gpu_util import to_host
    lr = 1e-2
    n = T * bag
    rows = torch.empty(n, dtype=torch.int32, device="cuda")
    nu = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(P.pkm_bag_backward_workspace_size(T, bag, cfg.N), dtype=torch.uint8, device="cuda")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    say("bag update full size")
    dw2 = torch.full((T, bag), float("nan"), device="cuda")
    ds2 = torch.full((T, bag), float("nan"), device="cuda")
    P.pkm_bag_backward(wl.values, cfg.N, cfg.d_v, cfg.dtype, dev(idx.astype(np.int32)), dev(w), dev(dy), T, bag,
                       dw=dw2, ds=ds2, softmax_group=cfg.k, rows=rows, n_unique=nu, update=True, lr=lr, workspace=ws)
    torch.cuda.synchronize()
    _check({"dw": dw2.cpu().numpy(), "ds": ds2.cpu().numpy()}, rows_of, cfg.N, idx, w.astype(np.float64),
           dy.astype(np.float64), cfg.k, tokens=tokens)
    assert int(nu.item()) == len(uniq)
    np.testing.assert_array_equal(rows[:len(uniq)].cpu().numpy(), uniq)
    for r in pick:
        pos = np.nonzero(flat_i == r)[0]
        g = np.sum(flat_w[pos, None] * dy[pos // bag].astype(np.float64), axis=0)
        ref = O.to_f64(wl.host_rows(np.array([r])), cfg.dtype)[0] - lr * g
        after = O.to_f64(to_host(wl.values[int(r)])[None], cfg.dtype)[0]
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        assert np.all(np.abs(after - ref) <= ulp + lr * 1e-4 * np.abs(g).max()), f"update of row {r}"
    untouched = np.setdiff1d(rng.integers(0, cfg.N, 64), uniq)
    got_u = to_host(wl.values[torch.from_numpy(untouched).cuda()])
    np.testing.assert_array_equal(np.asarray(got_u).view(np.uint8),
                                  np.asarray(wl.host_rows(untouched)).view(np.uint8))
    wl.close()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_one_row_table(dt):
    """n_rows = 1: every in-range entry hits the same row (one owner walks them all) and the
    sort works on one-bit keys; indices -1 and 1 read nothing."""
    from tests.gpu_util import to_dev, to_host
    rng = np.random.default_rng(31)
    n_rows, dim, n_bags, bag = 1, 64, 7, 6
    idx = rng.integers(-1, 2, size=(n_bags, bag))
    idx[0, 0] = 0
    w = rng.random((n_bags, bag)).astype(np.float32)
    dy = rng.standard_normal((n_bags, dim)).astype(np.float32)
    host = S.value_rows(19, np.arange(n_rows), dim, dt)
    table = to_dev(host, dt)
    lr = 0.25
    say(f"bag backward one-row table {dt}")
    got = _run(table, n_rows, dim, dt, idx, w, dy, 3, update=True, lr=lr)
    rows_of = lambda r: O.to_f64(host[np.asarray(r)], dt)
    _check(got, rows_of, n_rows, idx, w.astype(np.float64), dy.astype(np.float64), 3)
    np.testing.assert_array_equal(got["rows"], [0])
    _one_ulp(to_host(table)[[0]], O.to_f64(host[[0]], dt) - lr * got["grad"].astype(np.float64), dt)
