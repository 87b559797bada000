"""GPU parity of the k = 1 lookups and the shared memory pool, through the C ABI.

* Memory Attention token-memory values (summary of "Memory Attention": how it works,
  how it differs): the folded table against the oracle's float64 fold (one storage
  rounding), and V = K + E_bar[s] stage-wise from the GPU's own folded bytes (bitwise
  for fp32; bf16 within one ulp, almost always equal).
* Shared memory pool ("Memory Layers at Scale" digest, shared memory pool): several
  memory layers with their own query projections and gates over ONE value table, each
  checked against the oracle like a single layer.
"""

from __future__ import annotations

import gc
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle import ma as M  # noqa: E402
from oracle import pkm as O  # noqa: E402
from synth import CONFIGS  # noqa: E402
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


def _ma_case(cfg, seed, ids=None):
    import sparse_key_value_amd as P
    from tests.gpu_util import TORCH_DT, to_dev, to_host

    d = S.make_ma_inputs(cfg, seed)
    if ids is not None:
        d["ids"] = np.asarray(ids, dtype=np.int32)
        d["K"] = np.ascontiguousarray(S.normal_tensor(seed, S.TID_MA_KEYS, (len(ids), cfg.d_v), 1.0, cfg.dtype))
    T = len(d["ids"])
    E = to_dev(d["E"], cfg.dtype)
    Eb = torch.empty_like(E)
    gain = torch.from_numpy(d["gain"]).cuda() if d["gain"] is not None else None
    P.ma_fold_table(E, cfg.vocab, cfg.d_v, cfg.n_heads, gain, cfg.norm_eps, cfg.dtype, Eb)
    ids_d = torch.from_numpy(d["ids"]).cuda()
    K = to_dev(d["K"], cfg.dtype)
    V = torch.empty((T, cfg.d_v), dtype=TORCH_DT[cfg.dtype], device="cuda")
    P.ma_values(Eb, cfg.vocab, cfg.d_v, cfg.dtype, ids_d, T, K, V)
    # in place fold gives the same bytes
    E2 = E.clone()
    P.ma_fold_table(E2, cfg.vocab, cfg.d_v, cfg.n_heads, gain, cfg.norm_eps, cfg.dtype, E2)
    torch.cuda.synchronize()
    return d, to_host(Eb), to_host(E2), to_host(V)


def _check_ma(cfg, d, eb_gpu, eb_inplace, v_gpu):
    dt = cfg.dtype
    fold = M.fold_table(O.to_f64(d["E"], dt), cfg.n_heads, d["gain"], cfg.norm_eps)
    if dt == "bf16":
        PAR.check_bf16_rounded(eb_gpu, fold, 1e-6, "folded table")
    else:
        np.testing.assert_allclose(eb_gpu, fold, rtol=3e-6, atol=1e-7)
    np.testing.assert_array_equal(np.asarray(eb_gpu).view(np.uint8), np.asarray(eb_inplace).view(np.uint8))
    ref = M.values(eb_gpu, d["ids"], d["K"], dt)
    if dt == "bf16":
        PAR.check_bf16_rounded(v_gpu, ref, 0.0, "V = K + E_bar[s]")
        same = np.mean(v_gpu == M.store(ref, dt))
        assert same > 0.999, f"only {same:.4%} of V bitwise equal to the single rounding"
    else:
        np.testing.assert_array_equal(v_gpu, M.store(ref, dt))


@pytest.mark.parametrize("name", ["ma_tiny_f32", "ma_values_32k_bf16"])
def test_ma_values_match_oracle(name):
    cfg = C.MA_CONFIGS[name]
    say(f"memory attention {name}")
    _check_ma(cfg, *_ma_case(cfg, seed=4))


@pytest.mark.parametrize("shape", [dict(T=1), dict(T=257, gain=False), dict(dtype="bf16", d_v=64, n_heads=8, T=33)])
def test_ma_edge_shapes(shape):
    cfg = C.MA_CONFIGS["ma_tiny_f32"].with_(**shape)
    say(f"memory attention edge {shape}")
    _check_ma(cfg, *_ma_case(cfg, seed=6))


def test_ma_out_of_range_ids_read_no_row():
    cfg = C.MA_CONFIGS["ma_tiny_f32"]
    ids = [0, -1, cfg.vocab - 1, cfg.vocab, 1 << 30, 5]
    d, eb, eb2, v = _ma_case(cfg, seed=2, ids=ids)
    _check_ma(cfg, d, eb, eb2, v)
    for t in (1, 3, 4):
        np.testing.assert_array_equal(v[t], d["K"][t])


def test_shared_pool_three_layers_over_one_table():
    """Three memory layers (own W_q, sub-keys, W1, W2) read one value table."""
    from tests import gpu_util as G
    from tests.test_gpu_parity import full_check, run_debug

    cfg = CONFIGS["pkm_1m_bf16"].with_(memory_plus=True)
    T = 150
    before = torch.cuda.memory_allocated()
    first = G.Workload(cfg, seed=0, T=T)
    table_bytes = first.values.numel() * first.values.element_size()
    storage_bytes = first.values.untyped_storage().nbytes()   # with any alignment padding
    layers = [first] + [G.Workload(cfg, seed=s, T=T, values=first.values, value_seed=0) for s in (1, 2)]
    grown = torch.cuda.memory_allocated() - before
    # two more copies would add 2 x table_bytes; the handles' own workspaces are far smaller
    assert grown < storage_bytes + 0.5 * table_bytes, "each layer must borrow the pool, not copy it"
    for i, wl in enumerate(layers):
        say(f"shared pool layer {i}")
        assert wl.values.data_ptr() == first.values.data_ptr()
        full_check(wl, run_debug(wl))
    # the layers really differ (own projections) while reading the same rows' storage
    outs = [run_debug(wl)["idx"] for wl in layers]
    assert not np.array_equal(outs[0], outs[1])
    for wl in layers:
        wl.close()


def test_host_resident_value_table():
    """The value table in pinned host memory: the gather reads it over the host link; the
    forward and the EmbeddingBag give the same bytes as with the table in HBM."""
    import sparse_key_value_amd as P
    from tests import gpu_util as G

    cfg = CONFIGS["pkm_1m_bf16"].with_(memory_plus=True)
    T = 96
    dev = G.Workload(cfg, seed=0, T=T)
    host_v = torch.empty(dev.values.shape, dtype=dev.values.dtype, pin_memory=True)
    host_v.copy_(dev.values)
    torch.cuda.synchronize()
    hwl = G.Workload(cfg, seed=0, T=T, values=host_v, value_seed=0)
    x = dev.dev["x"]
    outs = []
    for wl in (dev, hwl):
        o = torch.empty((T, cfg.d_out), dtype=x.dtype, device="cuda")
        wl.pkm.forward(x, out=o)
        outs.append(G.to_host(o))
    np.testing.assert_array_equal(outs[0], outs[1])
    full_rows = [G.to_host(t) for t in (dev.values[:4], host_v[:4])]
    np.testing.assert_array_equal(full_rows[0], full_rows[1])
    # the EmbeddingBag over the host table, uniform indices
    idx, w = S.uniform_bags(3, 500, 16, cfg.N)
    idx_d, w_d = torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda()
    ys = []
    for table in (dev.values, host_v):
        y = torch.empty((500, cfg.d_v), dtype=torch.float32, device="cuda")
        P.pkm_embedding_bag(table, cfg.N, cfg.d_v, cfg.dtype, idx_d, w_d, 500, 16, y)
        ys.append(y.cpu().numpy())
    np.testing.assert_array_equal(ys[0], ys[1])
    ref = O.weighted_bag(lambda r: O.to_f64(S.value_rows(0, r, cfg.d_v, cfg.dtype), cfg.dtype),
                         idx.astype(np.int64), w.astype(np.float64))
    PAR.check_rows(ys[1], ref, 1e-4, "EmbeddingBag over the host table")
    # pageable host memory is refused
    with pytest.raises(P.PkmError):
        P.pkm_embedding_bag(torch.empty(16, cfg.d_v, dtype=dev.values.dtype), 16, cfg.d_v, cfg.dtype, idx_d, w_d,
                            1, 1, y)
    hwl.close()
    dev.close()


def test_values_in_a_hip_graph():
    """ma_values allocates nothing and never waits on the host: captured in a HIP graph, every
    replay equals the eager call bitwise, also after the captured ids change."""
    import sparse_key_value_amd as P
    from tests.gpu_util import TORCH_DT, to_dev
    cfg = C.MA_CONFIGS["ma_tiny_f32"]
    say("memory attention values in a HIP graph")
    d = S.make_ma_inputs(cfg, 9)
    T = len(d["ids"])
    E = to_dev(d["E"], cfg.dtype)
    gain = torch.from_numpy(d["gain"]).cuda() if d["gain"] is not None else None
    P.ma_fold_table(E, cfg.vocab, cfg.d_v, cfg.n_heads, gain, cfg.norm_eps, cfg.dtype, E)
    ids = torch.from_numpy(d["ids"]).cuda()
    ids_other = torch.flip(ids, [0]).contiguous()
    K = to_dev(d["K"], cfg.dtype)
    V = torch.empty((T, cfg.d_v), dtype=TORCH_DT[cfg.dtype], device="cuda")
    want = []
    for src in (ids.clone(), ids_other):
        out = torch.empty_like(V)
        P.ma_values(E, cfg.vocab, cfg.d_v, cfg.dtype, src, T, K, out)
        torch.cuda.synchronize()
        want.append(out)
    captured_ids = ids.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        P.ma_values(E, cfg.vocab, cfg.d_v, cfg.dtype, captured_ids, T, K, V)
    for rep, which in enumerate((0, 1, 0)):
        captured_ids.copy_(ids if which == 0 else ids_other)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(V, want[which]), f"replay {rep} differs from the eager call"
        P.ma_values(E, cfg.vocab, cfg.d_v, cfg.dtype, ids_other, T, K, torch.empty_like(V))
        torch.cuda.synchronize()
