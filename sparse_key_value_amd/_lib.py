"""ctypes binding of ``libpkm.so`` (the C ABI in ``include/pkm.h``, ``include/engram.h``,
``include/ma.h`` and ``include/bag_backward.h``).

Argument marshalling only: every function has the name of the C entry point it
calls, takes torch tensors (or raw device addresses as ints, or None for NULL)
and passes their data pointers and the current HIP stream.  No computation of
the forward happens in Python.  If the library has not been built this module
raises at import time; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkm.so")

PKM_OK, PKM_EINVAL, PKM_EUNSUPPORTED, PKM_EWORKSPACE, PKM_EHIP = 0, -1, -2, -3, -4
PKM_F32, PKM_BF16 = 0, 1
PKM_BOUND_AUTO, PKM_BOUND_EXACT = 0, 1
PKM_BAG_BACKWARD_NOALLOC_BYTES = 96 << 20   # the fixed sort buffers of pkm_bag_backward_noalloc (bag_backward.h)
STAGES = ["project", "qnorm", "score", "combine", "gather", "gate", "total"]
STAGE_ID = {n: i for i, n in enumerate(STAGES)}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python sparse_key_value_amd/build.py` "
                      "(the product-key memory path has no CPU fallback)")

_lib = ctypes.CDLL(LIB_PATH)


class pkm_config(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("d_query", ctypes.c_int32),
        ("n_sub", ctypes.c_int32), ("k", ctypes.c_int32), ("d_value", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("qk_norm", ctypes.c_int32), ("memory_plus", ctypes.c_int32),
        ("norm_eps", ctypes.c_float), ("max_tokens", ctypes.c_int64),
    ]


class pkm_debug_ptrs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("qhat", "half_idx", "half_score", "idx", "score", "w", "y", "theta",
                                               "counts")]


class engram_config(ctypes.Structure):
    _fields_ = [
        ("min_order", ctypes.c_int32), ("n_orders", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("table_rows", ctypes.c_int64), ("vocab", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("residual", ctypes.c_int32), ("norm_eps", ctypes.c_float),
    ]


class pkm_bag_backward_args(ctypes.Structure):
    _fields_ = [
        ("table", ctypes.c_void_p), ("n_rows", ctypes.c_int64), ("dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("idx", ctypes.c_void_p), ("w", ctypes.c_void_p), ("dy", ctypes.c_void_p), ("n_bags", ctypes.c_int64),
        ("bag_size", ctypes.c_int32), ("dw", ctypes.c_void_p), ("ds", ctypes.c_void_p),
        ("softmax_group", ctypes.c_int32), ("rows", ctypes.c_void_p), ("grad", ctypes.c_void_p),
        ("n_unique", ctypes.c_void_p), ("update", ctypes.c_int32), ("lr", ctypes.c_float),
    ]


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_sig = {
    "pkm_workspace_size": (_sz, [ctypes.POINTER(pkm_config)]),
    "pkm_create": (ctypes.c_int, [ctypes.POINTER(pkm_config), _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, ctypes.POINTER(_vp)]),
    "pkm_forward": (ctypes.c_int, [_vp, _vp, _i64, _vp, _vp, _vp, _vp]),
    "pkm_forward_debug": (ctypes.c_int, [_vp, _vp, _i64, _vp, ctypes.POINTER(pkm_debug_ptrs), _vp]),
    "pkm_select": (ctypes.c_int, [_vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "pkm_copy_normalized_subkeys": (ctypes.c_int, [_vp, _vp, _vp]),
    "pkm_embedding_bag": (ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, _vp, _i64, _i32, _vp, _vp]),
    "pkm_enable_stage_timing": (ctypes.c_int, [_vp, _i32]),
    "pkm_stage_times": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(ctypes.c_float), _i32]),
    "pkm_set_stage_timing_mask": (ctypes.c_int, [_vp, ctypes.c_uint32]),
    "pkm_set_score_bound": (ctypes.c_int, [_vp, _i32]),
    "pkm_destroy": (ctypes.c_int, [_vp]),
    "pkm_last_error": (ctypes.c_char_p, []),
    "engram_hash": (ctypes.c_int, [ctypes.POINTER(engram_config), _vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "engram_forward": (ctypes.c_int, [ctypes.POINTER(engram_config), _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp]),
    "engram_prefetch": (ctypes.c_int, [ctypes.POINTER(engram_config), _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "engram_forward_staged": (ctypes.c_int, [ctypes.POINTER(engram_config), _vp, _vp, _i64, _vp, _vp, _vp, _vp]),
    "pkm_bag_backward_workspace_size": (_sz, [_i64, _i32, _i64]),
    "pkm_bag_backward": (ctypes.c_int, [ctypes.POINTER(pkm_bag_backward_args), _vp, _sz, _vp]),
    "pkm_bag_backward_noalloc": (ctypes.c_int, [ctypes.POINTER(pkm_bag_backward_args), _vp]),
    "ma_fold_table": (ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, ctypes.c_float, _i32, _vp, _vp]),
    "ma_values": (ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, _i64, _vp, _vp, _vp]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype, _f.argtypes = _res, _args

EXPORTED = tuple(_sig)


class PkmError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where} failed with code {code}: {pkm_last_error()}")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None


def _check(rc: int, where: str) -> int:
    if rc < 0:
        raise PkmError(rc, where)
    return rc


def make_config(d_model, n_heads, d_query, n_sub, k, d_value, dtype, qk_norm, memory_plus, max_tokens,
                norm_eps=1e-6) -> pkm_config:
    dt = {"f32": PKM_F32, "bf16": PKM_BF16}.get(dtype, dtype)
    return pkm_config(int(d_model), int(n_heads), int(d_query), int(n_sub), int(k), int(d_value), int(dt),
                      int(bool(qk_norm)), int(bool(memory_plus)), float(norm_eps), int(max_tokens))


def pkm_last_error() -> str:
    return _lib.pkm_last_error().decode()


def pkm_workspace_size(cfg: pkm_config) -> int:
    n = _lib.pkm_workspace_size(ctypes.byref(cfg))
    if n == 0:
        code = PKM_EUNSUPPORTED if pkm_last_error().startswith("unsupported") else PKM_EINVAL
        raise PkmError(code, "pkm_workspace_size")
    return n


def pkm_create(cfg: pkm_config, W_q, subkeys, values, W1, W2, workspace, ws_bytes=None, stream=None) -> int:
    h = ctypes.c_void_p()
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.pkm_create(ctypes.byref(cfg), _ptr(W_q), _ptr(subkeys), _ptr(values), _ptr(W1), _ptr(W2),
                           _ptr(workspace), ws_bytes, _stream(stream), ctypes.byref(h)), "pkm_create")
    return h.value


def pkm_forward(h: int, x, T: int, out, idx_out=None, w_out=None, stream=None) -> None:
    _check(_lib.pkm_forward(h, _ptr(x), T, _ptr(out), _ptr(idx_out), _ptr(w_out), _stream(stream)), "pkm_forward")


def pkm_forward_debug(h: int, x, T: int, out, dbg: dict | None = None, stream=None) -> None:
    d = pkm_debug_ptrs(*[_ptr((dbg or {}).get(n)) for n, _ in pkm_debug_ptrs._fields_])
    _check(_lib.pkm_forward_debug(h, _ptr(x), T, _ptr(out), ctypes.byref(d), _stream(stream)), "pkm_forward_debug")


def pkm_select(h: int, qhat, T: int, half_idx=None, half_score=None, idx=None, score=None, w=None, stream=None) -> None:
    _check(_lib.pkm_select(h, _ptr(qhat), T, _ptr(half_idx), _ptr(half_score), _ptr(idx), _ptr(score), _ptr(w),
                           _stream(stream)), "pkm_select")


def pkm_copy_normalized_subkeys(h: int, dst, stream=None) -> None:
    _check(_lib.pkm_copy_normalized_subkeys(h, _ptr(dst), _stream(stream)), "pkm_copy_normalized_subkeys")


def pkm_embedding_bag(table, n_rows: int, dim: int, dtype, idx, w, n_bags: int, bag_size: int, y, stream=None) -> None:
    dt = {"f32": PKM_F32, "bf16": PKM_BF16}.get(dtype, dtype)
    _check(_lib.pkm_embedding_bag(_ptr(table), n_rows, dim, dt, _ptr(idx), _ptr(w), n_bags, bag_size, _ptr(y),
                                  _stream(stream)), "pkm_embedding_bag")


def pkm_enable_stage_timing(h: int, max_records: int) -> None:
    _check(_lib.pkm_enable_stage_timing(h, max_records), "pkm_enable_stage_timing")


def pkm_set_score_bound(h: int, mode) -> None:
    """PKM_BOUND_AUTO / "auto" (fp8 estimate where built) or PKM_BOUND_EXACT / "exact"."""
    m = {"auto": PKM_BOUND_AUTO, "exact": PKM_BOUND_EXACT}.get(mode, mode)
    _check(_lib.pkm_set_score_bound(h, int(m)), "pkm_set_score_bound")


def pkm_set_stage_timing_mask(h: int, stages) -> None:
    """Record only these stages (names from STAGES or ids) in the following forwards."""
    mask = 0
    for st in stages:
        mask |= 1 << (STAGE_ID[st] if isinstance(st, str) else int(st))
    _check(_lib.pkm_set_stage_timing_mask(h, mask), "pkm_set_stage_timing_mask")


def pkm_stage_times(h: int, stage, n: int) -> list[float]:
    sid = STAGE_ID.get(stage, stage)
    buf = (ctypes.c_float * max(1, n))()
    got = _check(_lib.pkm_stage_times(h, sid, buf, n), "pkm_stage_times")
    return [buf[i] for i in range(got)]


def pkm_destroy(h: int) -> None:
    _check(_lib.pkm_destroy(h), "pkm_destroy")


def make_engram_config(min_order, n_orders, n_heads, head_dim, table_rows, vocab, dtype, residual=False,
                       norm_eps=1e-6) -> engram_config:
    dt = {"f32": PKM_F32, "bf16": PKM_BF16}.get(dtype, dtype)
    return engram_config(int(min_order), int(n_orders), int(n_heads), int(head_dim), int(table_rows), int(vocab),
                         int(dt), int(bool(residual)), float(norm_eps))


def engram_hash(cfg: engram_config, ids, T: int, seq_len: int, compress, mult, rows, stream=None) -> None:
    _check(_lib.engram_hash(ctypes.byref(cfg), _ptr(ids), T, seq_len, _ptr(compress), _ptr(mult), _ptr(rows),
                            _stream(stream)), "engram_hash")


def engram_forward(cfg: engram_config, tables, ids, T: int, seq_len: int, compress, mult, h, out, e_out=None,
                   alpha_out=None, stream=None) -> None:
    _check(_lib.engram_forward(ctypes.byref(cfg), _ptr(tables), _ptr(ids), T, seq_len, _ptr(compress), _ptr(mult),
                               _ptr(h), _ptr(out), _ptr(e_out), _ptr(alpha_out), _stream(stream)), "engram_forward")


def engram_prefetch(cfg: engram_config, tables, ids, T: int, seq_len: int, compress, mult, staged, stream=None) -> None:
    _check(_lib.engram_prefetch(ctypes.byref(cfg), _ptr(tables), _ptr(ids), T, seq_len, _ptr(compress), _ptr(mult),
                                _ptr(staged), _stream(stream)), "engram_prefetch")


def engram_forward_staged(cfg: engram_config, staged, h, T: int, out, e_out=None, alpha_out=None, stream=None) -> None:
    _check(_lib.engram_forward_staged(ctypes.byref(cfg), _ptr(staged), _ptr(h), T, _ptr(out), _ptr(e_out),
                                      _ptr(alpha_out), _stream(stream)), "engram_forward_staged")


def ma_fold_table(E, vocab: int, d_v: int, n_heads: int, gain, eps: float, dtype, E_bar, stream=None) -> None:
    dt = {"f32": PKM_F32, "bf16": PKM_BF16}.get(dtype, dtype)
    _check(_lib.ma_fold_table(_ptr(E), vocab, d_v, n_heads, _ptr(gain), eps, dt, _ptr(E_bar), _stream(stream)),
           "ma_fold_table")


def ma_values(E_bar, vocab: int, d_v: int, dtype, ids, T: int, K, V, stream=None) -> None:
    dt = {"f32": PKM_F32, "bf16": PKM_BF16}.get(dtype, dtype)
    _check(_lib.ma_values(_ptr(E_bar), vocab, d_v, dt, _ptr(ids), T, _ptr(K), _ptr(V), _stream(stream)), "ma_values")


def pkm_bag_backward_workspace_size(n_bags: int, bag_size: int, n_rows: int) -> int:
    n = _lib.pkm_bag_backward_workspace_size(n_bags, bag_size, n_rows)
    if n == 0:
        raise PkmError(PKM_EINVAL, "pkm_bag_backward_workspace_size")
    return n


def pkm_bag_backward(table, n_rows: int, dim: int, dtype, idx, w, dy, n_bags: int, bag_size: int, dw=None, ds=None,
                     softmax_group: int = 0, rows=None, grad=None, n_unique=None, update: bool = False,
                     lr: float = 0.0, workspace=None, ws_bytes=None, stream=None) -> None:
    dt = {"f32": PKM_F32, "bf16": PKM_BF16}.get(dtype, dtype)
    a = pkm_bag_backward_args(_ptr(table), int(n_rows), int(dim), int(dt), _ptr(idx), _ptr(w), _ptr(dy), int(n_bags),
                              int(bag_size), _ptr(dw), _ptr(ds), int(softmax_group), _ptr(rows), _ptr(grad),
                              _ptr(n_unique), int(bool(update)), float(lr))
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.pkm_bag_backward(ctypes.byref(a), _ptr(workspace), ws_bytes, _stream(stream)), "pkm_bag_backward")


def pkm_bag_backward_noalloc(table, n_rows: int, dim: int, dtype, idx, w, dy, n_bags: int, bag_size: int, dw=None,
                             ds=None, softmax_group: int = 0, rows=None, grad=None, n_unique=None,
                             update: bool = False, lr: float = 0.0, stream=None) -> None:
    dt = {"f32": PKM_F32, "bf16": PKM_BF16}.get(dtype, dtype)
    a = pkm_bag_backward_args(_ptr(table), int(n_rows), int(dim), int(dt), _ptr(idx), _ptr(w), _ptr(dy), int(n_bags),
                              int(bag_size), _ptr(dw), _ptr(ds), int(softmax_group), _ptr(rows), _ptr(grad),
                              _ptr(n_unique), int(bool(update)), float(lr))
    _check(_lib.pkm_bag_backward_noalloc(ctypes.byref(a), _stream(stream)), "pkm_bag_backward_noalloc")
