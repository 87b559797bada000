"""The bag backward without a workspace argument (pkm_bag_backward_noalloc), through the C ABI,
against the entry point that takes a caller workspace (pkm_bag_backward).

Both run the same kernels, so every output is compared bitwise: dw, ds, the distinct rows and
their count, the row gradients and the updated table.  Two calls in a row, the second on a
smaller input, show that what the first call leaves in the library's fixed buffers does not
leak into the next.  A size whose sort buffers exceed the fixed array is refused before any
work is enqueued.
"""

from __future__ import annotations

import gc
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from synth import inputs as S  # noqa: E402


def say(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _case(dt, n_rows, dim, n_bags, H, k, seed):
    rng = np.random.default_rng(seed)
    bag = H * k
    idx = rng.integers(-2, n_rows + 2, size=(n_bags, bag)).astype(np.int32)   # a few read nothing
    idx[: n_bags // 4, :3] = 5                                              # a row many times, also within a bag
    s = rng.standard_normal((n_bags, H, k))
    w = np.exp(s - s.max(-1, keepdims=True))
    w = (w / w.sum(-1, keepdims=True)).reshape(n_bags, bag).astype(np.float32)
    dy = rng.standard_normal((n_bags, dim)).astype(np.float32)
    table = S.value_rows(seed, np.arange(n_rows), dim, dt)
    return dict(dt=dt, n_rows=n_rows, dim=dim, n_bags=n_bags, bag=bag, group=k, idx=idx, w=w, dy=dy, table=table)


def _call(c, noalloc, update, table):
    import sparse_key_value_amd as P
    n_bags, bag, dim = c["n_bags"], c["bag"], c["dim"]
    n = n_bags * bag
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = {"dw": torch.full((n_bags, bag), float("nan"), device="cuda"),
           "ds": torch.full((n_bags, bag), float("nan"), device="cuda"),
           "rows": torch.full((n,), -7, dtype=torch.int32, device="cuda"),
           "grad": torch.full((n, dim), float("nan"), device="cuda"),
           "n_unique": torch.full((1,), -1, dtype=torch.int32, device="cuda")}
    args = (table, c["n_rows"], dim, c["dt"], dev(c["idx"]), dev(c["w"]), dev(c["dy"]), n_bags, bag)
    kw = dict(softmax_group=c["group"], update=update, lr=0.25, **out)
    if noalloc:
        P.pkm_bag_backward_noalloc(*args, **kw)
    else:
        ws = torch.empty(P.pkm_bag_backward_workspace_size(n_bags, bag, c["n_rows"]), dtype=torch.uint8, device="cuda")
        P.pkm_bag_backward(*args, workspace=ws, **kw)
    torch.cuda.synchronize()
    u = int(out["n_unique"].item())
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["rows"], res["grad"] = res["rows"][:u], res["grad"][:u]
    return res


@pytest.mark.parametrize("update", [False, True])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_noalloc_backward_equals_the_workspace_entry_point(dt, update):
    from tests.gpu_util import to_dev, to_host
    # the second call is smaller in every dimension of the sort
    cases = [_case(dt, 5000, 256, 700, 4, 32, seed=1), _case(dt, 900, 64, 90, 2, 8, seed=2)]
    for i, c in enumerate(cases):
        say(f"noalloc backward {dt} update={update} call {i}: {c['n_bags']} bags x {c['bag']}, "
            f"{c['n_rows']} rows x {c['dim']}")
        tables = [to_dev(c["table"], dt) for _ in range(2)]
        ref = _call(c, False, update, tables[0])
        got = _call(c, True, update, tables[1])
        assert got["n_unique"][0] == ref["n_unique"][0] > 0
        for key in ("dw", "ds", "rows", "grad"):
            np.testing.assert_array_equal(got[key].view(np.uint8), ref[key].view(np.uint8), err_msg=key)
        after = [to_host(t) for t in tables]
        np.testing.assert_array_equal(after[1].view(np.uint8), after[0].view(np.uint8))
        if update:
            assert not np.array_equal(after[0].view(np.uint8), c["table"].view(np.uint8)), "the update changed nothing"


def test_noalloc_backward_refuses_sizes_beyond_its_buffers():
    """2^27 entries need far more sort buffers than the fixed array holds: PKM_EWORKSPACE, and
    nothing is enqueued (dw keeps its fill).  Every buffer has its full size, so even a launch
    would stay in bounds."""
    import sparse_key_value_amd as P
    # the stated capacity: 2^21 entries (16,384 tokens x 4 heads x 32) over any table
    for rows in (1 << 20, 1 << 26, (1 << 31) - 1):
        need = P.pkm_bag_backward_workspace_size(16384, 128, rows)
        say(f"sort buffers for 2^21 entries over {rows} rows: {need} bytes")
        assert need <= P.PKM_BAG_BACKWARD_NOALLOC_BYTES
    n_bags, bag, dim, n_rows = 1 << 16, 2048, 16, 64
    assert P.pkm_bag_backward_workspace_size(n_bags, bag, n_rows) > P.PKM_BAG_BACKWARD_NOALLOC_BYTES
    table = torch.zeros((n_rows, dim), dtype=torch.float32, device="cuda")
    idx = torch.zeros((n_bags, bag), dtype=torch.int32, device="cuda")
    w = torch.zeros((n_bags, bag), dtype=torch.float32, device="cuda")
    dy = torch.zeros((n_bags, dim), dtype=torch.float32, device="cuda")
    dw = torch.full((n_bags, bag), float("nan"), device="cuda")
    with pytest.raises(P.PkmError) as e:
        P.pkm_bag_backward_noalloc(table, n_rows, dim, "f32", idx, w, dy, n_bags, bag, dw=dw, update=True, lr=1.0)
    assert e.value.code == P.PKM_EWORKSPACE and "fixed" in str(e.value)
    torch.cuda.synchronize()
    assert bool(torch.isnan(dw).all())
    assert bool((table == 0).all())
