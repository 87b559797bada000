"""The C ABI on the CPU: the libraries load, export every declared entry point, and
reject bad arguments before touching a device (no compute calls here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header):
    txt = open(os.path.join(ROOT, "include", header)).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b((?:pkm|engram|ma)_[a-z_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def P():
    import sparse_key_value_amd as P
    return P


def test_library_exports_every_declared_symbol(P):
    lib = ctypes.CDLL(P.LIB_PATH)
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == ["bag_backward.h", "engram.h", "ma.h", "pkm.h"]
    names = sorted(set(n for hd in headers for n in _declared(hd)))
    assert {"pkm_create", "pkm_forward", "pkm_destroy", "pkm_embedding_bag", "engram_hash", "engram_forward",
            "ma_fold_table", "ma_values", "pkm_bag_backward", "pkm_bag_backward_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/pkm.h but not exported"
    assert set(names) == set(P.EXPORTED), "binding and header disagree"


def test_synth_library_exports():
    from synth import device as SD
    for n in ("synth_fill_values", "synth_stream_read", "synth_copy"):
        assert hasattr(SD._lib, n)


def _cfg(P, **kw):
    base = dict(d_model=2048, n_heads=4, d_query=512, n_sub=4096, k=32, d_value=2048, dtype="bf16", qk_norm=1,
                memory_plus=1, max_tokens=16384)
    base.update(kw)
    return P.make_config(**base)


def test_workspace_size_matches_layout(P):
    c = _cfg(P)
    a = lambda v: (v + 255) // 256 * 256
    T, H, dq, dm, dv, n, k = 16384, 4, 512, 2048, 2048, 4096, 32
    # the projection's output [T, H dq + dv] (q, then z) is stored in bf16
    want = (a(H * dq * dm * 2) + a(H * 2 * n * dq // 2 * 2) + a(dv * dm * 2) + a(dm * dv * 2) + a(T * H * dq * 2) +
            a(T * H * dq * 2) + a(T * H * 2 * 128 * 4) + a(T * H * 2 * 4) + a(T * H * 2 * 128 * 8) + a(T * H * 2 * 2 * 4) +
            2 * a(T * H * 2 * k * 4) + 3 * a(T * H * k * 4) + a(T * dv * 2) + a(T * dv * 2))
    # the fp8 bound (bf16, 256-wide halves): e4m3 sub-keys, their norms, the largest per (head,
    # half), e4m3 query halves and their norms
    want += a(H * 2 * n * 256) + a(H * 2 * n * 4) + a(H * 2 * 4) + a(T * H * 2 * 256) + a(T * H * 2 * 4)
    assert P.pkm_workspace_size(c) == want
    # without the gate there is no W1/W2 copy and no y/g buffer
    assert P.pkm_workspace_size(_cfg(P, memory_plus=0)) < want


@pytest.mark.parametrize("bad,needle", [
    (dict(dtype=7), "dtype"),
    (dict(d_model=0), "d_model"),
    (dict(d_model=1020), "d_model"),
    (dict(n_heads=0), "n_heads"),
    (dict(d_query=511), "d_query"),
    (dict(n_sub=0), "n_sub"),
    (dict(n_sub=46341), "2^31"),
    (dict(k=0), "k must"),
    (dict(k=65), "k must"),
    (dict(k=64, n_sub=63), "k must"),
    (dict(k=9, n_sub=8), "k must"),
    (dict(d_value=12), "d_value"),
    (dict(d_model=65536 + 32), "d_model must be <= 65536"),     # weight transposes: grid y of 32-row tiles
    (dict(d_value=65536 + 32), "d_value must be <= 65536"),
    (dict(qk_norm=2), "qk_norm"),
    (dict(max_tokens=0), "max_tokens"),
    (dict(max_tokens=1 << 25), "max_tokens"),
    (dict(max_tokens=1 << 23, n_heads=4), "max_tokens * n_heads"),   # 2^25 selection rows of 64 lanes
])
def test_invalid_configs_are_rejected(P, bad, needle):
    c = _cfg(P)
    for key, v in bad.items():
        setattr(c, key, v)
    with pytest.raises(P.PkmError) as e:
        P.pkm_workspace_size(c)
    assert needle in str(e.value)
    rc = P._lib._lib.pkm_create(ctypes.byref(c), 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 40, None,
                                ctypes.byref(ctypes.c_void_p()))
    assert rc == P.PKM_EINVAL and needle in P.pkm_last_error()


@pytest.mark.parametrize("d_query,k", [(96, 32), (6, 3), (130, 48), (512, 64), (2, 1), (258, 33)])
def test_workspace_of_padded_query_halves_and_wide_k(P, d_query, k):
    """Any even d_query up to 512 and any k up to 64: query halves and sub-key rows are stored
    padded to the next scoring width (64, 128 or 256), and k > 32 takes 256 candidate slots
    per row instead of 128."""
    a = lambda v: (v + 255) // 256 * 256
    T, H, dm, dv, n = 1000, 3, 256, 128, 700
    c = _cfg(P, d_query=d_query, k=k, n_heads=H, d_model=dm, d_value=dv, n_sub=n, max_tokens=T, memory_plus=0)
    d_h = d_query // 2
    dhp = 64 if d_h <= 64 else (128 if d_h <= 128 else 256)
    cs = 128 if k <= 32 else 256
    want = (a(H * d_query * dm * 2) + a(H * 2 * n * dhp * 2) + a(T * H * d_query * 2) + a(T * H * 2 * dhp * 2) +
            a(T * H * 2 * 128 * 4) + a(T * H * 2 * 4) + a(T * H * 2 * cs * 8) + a(T * H * 2 * 2 * 4) +
            2 * a(T * H * 2 * k * 4) + 3 * a(T * H * k * 4))
    if dhp == 256:   # the fp8 bound of bf16 workloads
        want += a(H * 2 * n * 256) + a(H * 2 * n * 4) + a(H * 2 * 4) + a(T * H * 2 * 256) + a(T * H * 2 * 4)
    assert P.pkm_workspace_size(c) == want


def test_query_halves_wider_than_the_scoring_kernels_are_unsupported(P):
    """d_query = 514 is a valid config (even) that the scoring kernels are not built for:
    PKM_EUNSUPPORTED, not PKM_EINVAL."""
    c = _cfg(P, d_query=514)
    with pytest.raises(P.PkmError) as e:
        P.pkm_workspace_size(c)
    assert e.value.code == P.PKM_EUNSUPPORTED and "256" in str(e.value)
    rc = P._lib._lib.pkm_create(ctypes.byref(c), 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 40, None,
                                ctypes.byref(ctypes.c_void_p()))
    assert rc == P.PKM_EUNSUPPORTED
    assert P.pkm_workspace_size(_cfg(P, d_query=512)) > 0


def test_create_argument_errors_before_any_device_call(P):
    c = _cfg(P)
    lib = P._lib._lib
    h = ctypes.c_void_p()
    assert lib.pkm_create(ctypes.byref(c), None, 256, 256, 256, 256, 256, 1 << 40, None, ctypes.byref(h)) == P.PKM_EINVAL
    assert lib.pkm_create(ctypes.byref(c), 256, 256, 256, None, 256, 256, 1 << 40, None, ctypes.byref(h)) == P.PKM_EINVAL
    assert "W1 and W2" in P.pkm_last_error()
    assert lib.pkm_create(ctypes.byref(c), 256, 256, 8, 256, 256, 256, 1 << 40, None, ctypes.byref(h)) == P.PKM_EINVAL
    assert "16-byte" in P.pkm_last_error()
    assert lib.pkm_create(ctypes.byref(c), 256, 256, 256, 256, 256, 256, 1024, None, ctypes.byref(h)) == P.PKM_EWORKSPACE
    assert lib.pkm_create(ctypes.byref(c), 256, 256, 256, 256, 256, 256, 1 << 40, None, None) == P.PKM_EINVAL


def test_other_entry_points_reject_bad_arguments(P):
    lib = P._lib._lib
    assert lib.pkm_forward(None, 256, 4, 256, None, None, None) == P.PKM_EINVAL
    assert lib.pkm_forward_debug(None, 256, 4, 256, None, None) == P.PKM_EINVAL
    assert lib.pkm_select(None, 256, 4, None, None, None, None, None, None) == P.PKM_EINVAL
    assert lib.pkm_destroy(None) == P.PKM_EINVAL
    assert lib.pkm_enable_stage_timing(None, 4) == P.PKM_EINVAL
    assert lib.pkm_set_stage_timing_mask(None, 1) == P.PKM_EINVAL
    assert lib.pkm_copy_normalized_subkeys(None, 256, None) == P.PKM_EINVAL
    eb = lib.pkm_embedding_bag
    assert eb(256, 10, 12, 1, 256, 256, 4, 4, 256, None) == P.PKM_EINVAL   # 12 bf16 = 24 bytes per row
    assert eb(256, 10, 16, 3, 256, 256, 4, 4, 256, None) == P.PKM_EINVAL   # bad dtype
    assert eb(256, 0, 16, 1, 256, 256, 4, 4, 256, None) == P.PKM_EINVAL    # no rows
    assert eb(256, 10, (1 << 24) + 8, 1, 256, 256, 4, 4, 256, None) == P.PKM_EINVAL  # wider than 2^24
    assert "2^24" in P.pkm_last_error()
    assert eb(256, 10, 16, 1, 256, 256, 4, 0, 256, None) == P.PKM_EINVAL   # empty bags
    assert eb(None, 10, 16, 1, 256, 256, 4, 4, 256, None) == P.PKM_EINVAL  # NULL table
    assert eb(8, 10, 16, 1, 256, 256, 4, 4, 256, None) == P.PKM_EINVAL     # misaligned table
    assert eb(None, 10, 16, 1, None, None, 0, 4, None, None) == P.PKM_OK   # zero bags: nothing to do


def _ecfg(P, **kw):
    base = dict(min_order=2, n_orders=2, n_heads=8, head_dim=128, table_rows=2097143, vocab=128000, dtype="bf16")
    base.update(kw)
    return P.make_engram_config(**base)


@pytest.mark.parametrize("bad,needle", [
    (dict(dtype=5), "dtype"),
    (dict(min_order=0), "min_order"),
    (dict(n_orders=0), "n_orders"),
    (dict(n_orders=5), "n_orders"),
    (dict(min_order=6, n_orders=4), "largest order"),
    (dict(n_heads=65), "n_heads"),
    (dict(head_dim=4), "head_dim"),
    (dict(head_dim=512), "4096 bytes"),
    (dict(table_rows=0), "table_rows"),
    (dict(table_rows=1 << 27), "2^31"),
    (dict(vocab=0), "vocab"),
    (dict(residual=2), "residual"),
    (dict(norm_eps=-1.0), "norm_eps"),
])
def test_engram_invalid_configs_are_rejected(P, bad, needle):
    c = _ecfg(P)
    for key, v in bad.items():
        setattr(c, key, v)
    lib = P._lib._lib
    assert lib.engram_hash(ctypes.byref(c), 256, 4, 4, None, 256, 256, None) == P.PKM_EINVAL
    assert needle in P.pkm_last_error()
    assert lib.engram_forward(ctypes.byref(c), 256, 256, 4, 4, None, 256, 256, 256, None, None, None) == P.PKM_EINVAL
    assert needle in P.pkm_last_error()


def test_engram_argument_errors_before_any_device_call(P):
    c = _ecfg(P)
    lib = P._lib._lib
    assert lib.engram_hash(None, 256, 4, 4, None, 256, 256, None) == P.PKM_EINVAL
    assert lib.engram_hash(ctypes.byref(c), 256, -1, 4, None, 256, 256, None) == P.PKM_EINVAL
    assert lib.engram_hash(ctypes.byref(c), 256, 4, 0, None, 256, 256, None) == P.PKM_EINVAL
    assert "seq_len" in P.pkm_last_error()
    assert lib.engram_hash(ctypes.byref(c), None, 4, 4, None, 256, 256, None) == P.PKM_EINVAL
    assert lib.engram_hash(ctypes.byref(c), 256, 4, 4, None, 256, None, None) == P.PKM_EINVAL
    assert lib.engram_forward(ctypes.byref(c), None, 256, 4, 4, None, 256, 256, 256, None, None, None) == P.PKM_EINVAL
    assert lib.engram_forward(ctypes.byref(c), 256, 256, 4, 4, None, 256, 264, 256, None, None, None) == P.PKM_EINVAL
    assert "16-byte" in P.pkm_last_error()
    pf, st = lib.engram_prefetch, lib.engram_forward_staged
    assert pf(ctypes.byref(c), None, 256, 4, 4, None, 256, 256, None) == P.PKM_EINVAL
    assert pf(ctypes.byref(c), 256, 256, 4, 4, None, 256, 8, None) == P.PKM_EINVAL and "16-byte" in P.pkm_last_error()
    assert st(ctypes.byref(c), None, 256, 4, 256, None, None, None) == P.PKM_EINVAL
    assert st(ctypes.byref(c), 256, 256, 4, 256, 8, None, None) == P.PKM_EINVAL and "16-byte" in P.pkm_last_error()
    assert pf(ctypes.byref(c), None, None, 0, 4, None, None, None, None) == P.PKM_OK
    assert st(ctypes.byref(c), None, None, 0, None, None, None, None) == P.PKM_OK
    # T = 0 is a no-op that needs no pointers
    assert lib.engram_hash(ctypes.byref(c), None, 0, 4, None, None, None, None) == P.PKM_OK
    assert lib.engram_forward(ctypes.byref(c), None, None, 0, 4, None, None, None, None, None, None, None) == P.PKM_OK


def test_ma_argument_errors_before_any_device_call(P):
    lib = P._lib._lib
    f, v = lib.ma_fold_table, lib.ma_values
    assert f(256, 10, 64, 4, None, 1e-6, 2, 256, None) == P.PKM_EINVAL and "dtype" in P.pkm_last_error()
    assert f(256, 10, 12, 1, None, 1e-6, 1, 256, None) == P.PKM_EINVAL and "d_v" in P.pkm_last_error()
    assert f(256, 10, 64, 3, None, 1e-6, 1, 256, None) == P.PKM_EINVAL and "n_heads" in P.pkm_last_error()
    assert f(256, 10, 64, 16, None, 1e-6, 1, 256, None) == P.PKM_EINVAL   # 4 bf16 per head = 8 bytes
    assert f(256, 10, 64, 4, None, -1.0, 1, 256, None) == P.PKM_EINVAL and "eps" in P.pkm_last_error()
    assert f(None, 10, 64, 4, None, 1e-6, 1, 256, None) == P.PKM_EINVAL
    assert f(8, 10, 64, 4, None, 1e-6, 1, 256, None) == P.PKM_EINVAL and "aligned" in P.pkm_last_error()
    assert f(None, 0, 64, 4, None, 1e-6, 1, None, None) == P.PKM_OK
    assert v(256, 0, 64, 1, 256, 4, 256, 256, None) == P.PKM_EINVAL and "vocab" in P.pkm_last_error()
    assert v(256, 10, 64, 1, None, 4, 256, 256, None) == P.PKM_EINVAL
    assert v(256, 10, 64, 1, 256, -1, 256, 256, None) == P.PKM_EINVAL
    assert v(256, 10, 64, 1, 256, 4, 264, 256, None) == P.PKM_EINVAL and "aligned" in P.pkm_last_error()
    assert v(None, 10, 64, 1, None, 0, None, None, None) == P.PKM_OK


def test_bag_backward_argument_errors_before_any_device_call(P):
    lib = P._lib._lib
    assert lib.pkm_bag_backward(None, None, 0, None) == P.PKM_EINVAL
    assert lib.pkm_bag_backward_workspace_size(-1, 4, 100) == 0
    assert lib.pkm_bag_backward_workspace_size(10, 0, 100) == 0 and "bag_size" in P.pkm_last_error()
    assert lib.pkm_bag_backward_workspace_size(10, 4096, 100) == 0
    assert lib.pkm_bag_backward_workspace_size(1 << 23, 512, 100) == 0 and "2^31" in P.pkm_last_error()
    # one block per bag: 2^24 bags of 256 lanes would exceed a dispatch's 2^32 work-items
    assert lib.pkm_bag_backward_workspace_size(1 << 24, 1, 100) == 0 and "2^24" in P.pkm_last_error()
    assert lib.pkm_bag_backward_workspace_size(10, 4, 0) == 0 and "n_rows" in P.pkm_last_error()

    def args(**kw):
        base = dict(table=256, n_rows=100, dim=64, dtype=1, idx=256, w=256, dy=256, n_bags=4, bag_size=8)
        base.update(kw)
        return P.pkm_bag_backward_args(**base)

    bb = lambda a: lib.pkm_bag_backward(ctypes.byref(a), None, 0, None)
    assert bb(args(dtype=3)) == P.PKM_EINVAL and "dtype" in P.pkm_last_error()
    assert bb(args(dim=4)) == P.PKM_EINVAL and "dim" in P.pkm_last_error()
    assert bb(args(dim=4096)) == P.PKM_EINVAL
    assert bb(args(ds=256, softmax_group=3)) == P.PKM_EINVAL and "softmax_group" in P.pkm_last_error()
    assert bb(args(update=2)) == P.PKM_EINVAL
    assert bb(args(table=None)) == P.PKM_EINVAL
    assert bb(args(dy=8)) == P.PKM_EINVAL and "aligned" in P.pkm_last_error()
    assert bb(args(n_bags=0, table=None, idx=None, w=None, dy=None)) == P.PKM_OK
    # the entry point without a workspace checks the same arguments before touching the device
    na = lambda a: lib.pkm_bag_backward_noalloc(ctypes.byref(a), None)
    assert lib.pkm_bag_backward_noalloc(None, None) == P.PKM_EINVAL
    assert na(args(dtype=3)) == P.PKM_EINVAL and "dtype" in P.pkm_last_error()
    assert na(args(n_bags=1 << 24)) == P.PKM_EINVAL and "2^24" in P.pkm_last_error()
    assert na(args(dy=8)) == P.PKM_EINVAL and "aligned" in P.pkm_last_error()
    assert na(args(n_bags=0, table=None, idx=None, w=None, dy=None)) == P.PKM_OK
    # the binding's size of the fixed buffers is the header's
    import re
    hdr = open(os.path.join(ROOT, "include", "bag_backward.h")).read()
    m = re.search(r"#define PKM_BAG_BACKWARD_NOALLOC_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == P.PKM_BAG_BACKWARD_NOALLOC_BYTES


def test_python_class_checks_tensor_shapes_before_any_call(P):
    """The C ABI takes bare pointers, so ProductKeyMemory checks every tensor's shape, type,
    layout and device before a kernel could read past the end of one."""
    import torch

    bf = torch.bfloat16
    good = dict(W_q=torch.zeros(64, 2 * 16, dtype=bf), subkeys=torch.zeros(2, 2, 8, 8, dtype=bf),
                values=torch.zeros(64, 32, dtype=bf), W1=torch.zeros(64, 32, dtype=bf), W2=torch.zeros(32, 64, dtype=bf))
    cfg = dict(d_model=64, n_heads=2, d_query=16, n_sub=8, k=4, d_value=32, dtype="bf16", qk_norm=1, memory_plus=1,
               max_tokens=16)
    cases = [("W_q", torch.zeros(64, 16, dtype=bf), "shape"),
             ("subkeys", torch.zeros(2, 2, 8, 8, dtype=torch.float32), "dtype"),
             ("values", torch.zeros(32, 64, dtype=bf).t(), "contiguous"),
             ("W2", torch.zeros(32, 32, dtype=bf), "shape"),
             ("W1", None, "torch tensor")]
    for name, t, needle in cases:
        kw = dict(good, **{name: t})
        with pytest.raises(ValueError) as e:
            P.ProductKeyMemory(**cfg, **kw)
        assert name in str(e.value) and needle in str(e.value)
    with pytest.raises(ValueError) as e:   # right shapes, but host memory that is not pinned
        P.ProductKeyMemory(**cfg, **good)
    assert "W_q must be on the GPU" in str(e.value)
    from sparse_key_value_amd import _check_tensor
    with pytest.raises(ValueError, match="x has shape"):
        _check_tensor("x", torch.zeros(5, 32, dtype=bf), (5, 64), bf)
