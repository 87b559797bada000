"""ctypes wrapper of ``synth/libpkm_synth.so``: GPU-side input generation and
bandwidth-reference kernels for tests and benchmarks (not the product path)."""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkm_synth.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python sparse_key_value_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)
_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
_lib.synth_fill_values.argtypes = [_vp, _i64, _i64, _i32, _i32, ctypes.c_uint64, _vp]
_lib.synth_fill_table.argtypes = [_vp, _i64, _i64, _i32, _i32, ctypes.c_uint64, ctypes.c_uint32, _vp]
_lib.synth_stream_read.argtypes = [_vp, _i64, _vp, _i32, _vp]
_lib.synth_copy.argtypes = [_vp, _vp, _i64, _i32, _vp]
_lib.synth_row_read.argtypes = [_vp, _i64, _i64, _vp, _i64, _i32, _vp, _vp]
for _f in (_lib.synth_fill_values, _lib.synth_fill_table, _lib.synth_stream_read, _lib.synth_copy, _lib.synth_row_read):
    _f.restype = ctypes.c_int


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def fill_values(table, seed: int, row0: int = 0, n_rows: int | None = None, tid: int = 6) -> None:
    """Fill rows of a [N, d_v] torch tensor (float32 or bfloat16) on the GPU from the
    row-addressable stream of tensor id ``tid`` (6: the value table)."""
    import torch
    dt = 1 if table.dtype == torch.bfloat16 else 0
    n_rows = table.shape[0] - row0 if n_rows is None else n_rows
    rc = _lib.synth_fill_table(table.data_ptr(), row0, n_rows, table.shape[1], dt, seed, tid, _stream())
    if rc:
        raise RuntimeError(f"synth_fill_table failed: hip error {rc}")


def fill_rows(buf, seed: int, row0: int, n_rows: int, tid: int = 6) -> None:
    """Fill buf[0:n_rows] with rows row0 .. row0 + n_rows - 1 of the table of tensor id ``tid``
    (a piece of a table too large to keep on the GPU)."""
    import torch
    assert 0 <= n_rows <= buf.shape[0]
    dt = 1 if buf.dtype == torch.bfloat16 else 0
    row_bytes = buf.shape[1] * buf.element_size()
    # the generator addresses rows from the table's row 0; only rows row0 .. row0 + n_rows - 1,
    # i.e. buf[0:n_rows], are written
    rc = _lib.synth_fill_table(buf.data_ptr() - row0 * row_bytes, row0, n_rows, buf.shape[1], dt, seed, tid,
                               _stream())
    if rc:
        raise RuntimeError(f"synth_fill_table failed: hip error {rc}")


def stream_read(buf, sink, grid: int = 2048) -> None:
    rc = _lib.synth_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), grid, _stream())
    if rc:
        raise RuntimeError(f"synth_stream_read failed: hip error {rc}")


def copy(dst, src, grid: int = 2048) -> None:
    rc = _lib.synth_copy(dst.data_ptr(), src.data_ptr(), src.numel() * src.element_size(), grid, _stream())
    if rc:
        raise RuntimeError(f"synth_copy failed: hip error {rc}")


def row_read(table, idx, out) -> None:
    """Read the rows of ``table`` ([N, *] on the GPU) that the bags of ``idx`` ([n_bags, bag]
    int32) name, with a weighted bag gather's lane layout and no arithmetic but an XOR:
    out[b] (``table.shape[1:]`` bytes per bag) = the XOR of the bag's rows, bytewise.
    Indices outside [0, N) read row 0."""
    import torch
    assert idx.dtype == torch.int32 and idx.dim() == 2 and idx.is_contiguous() and table.is_contiguous()
    row_bytes = table[0].numel() * table.element_size()
    assert out.is_contiguous() and out.numel() * out.element_size() == idx.shape[0] * row_bytes
    rc = _lib.synth_row_read(table.data_ptr(), table.shape[0], row_bytes, idx.data_ptr(), idx.shape[0], idx.shape[1],
                             out.data_ptr(), _stream())
    if rc:
        raise RuntimeError(f"synth_row_read failed: hip error {rc}")
