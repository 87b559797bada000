"""Product-key memory forward for AMD Instinct MI355X (gfx950).

The forward ("Memory Layers at Scale": a product-key memory layer in place of an
FFN) runs entirely in the HIP kernels of ``libpkm.so`` behind the C ABI of
``include/pkm.h``, and so does the hashed n-gram lookup (Engram review: multi-head
hashing and the context-aware gate) behind ``include/engram.h`` and the Memory
Attention token-memory values (V = K + folded table row) behind ``include/ma.h`` and the
EmbeddingBag backward with the sparse update behind ``include/bag_backward.h``; this package only
marshals arguments (``_lib``) and manages device memory with PyTorch
(``ProductKeyMemory``).
"""

from __future__ import annotations

from ._lib import (  # noqa: F401
    EXPORTED, LIB_PATH, PKM_BAG_BACKWARD_NOALLOC_BYTES, PKM_BF16, PKM_BOUND_AUTO, PKM_BOUND_EXACT, PKM_EHIP, PKM_EINVAL, PKM_EUNSUPPORTED, PKM_EWORKSPACE, PKM_F32, PKM_OK, STAGES,
    PkmError, make_config, pkm_config, pkm_copy_normalized_subkeys, pkm_create, pkm_debug_ptrs, pkm_destroy,
    pkm_embedding_bag, pkm_enable_stage_timing, pkm_forward, pkm_forward_debug, pkm_last_error, pkm_select,
    pkm_set_score_bound, pkm_set_stage_timing_mask, pkm_stage_times, pkm_workspace_size,
    engram_config, engram_forward, engram_forward_staged, engram_hash, engram_prefetch, make_engram_config,
    ma_fold_table, ma_values, pkm_bag_backward, pkm_bag_backward_args, pkm_bag_backward_noalloc, pkm_bag_backward_workspace_size,
)


def _check_tensor(name, t, shape, dtype, host_ok=False, device=True):
    """A contiguous torch tensor of exactly `shape` and `dtype`, on a GPU (or, with host_ok, in
    pinned host memory; device=False: any device); ValueError otherwise."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    if device and not (t.is_cuda or (host_ok and t.is_pinned())):
        raise ValueError(f"{name} must be on the GPU" + (" or in pinned host memory" if host_ok else ""))


class ProductKeyMemory:
    """Owns a handle and its workspace (a torch uint8 tensor on the current device).

    Tensors (torch, on the GPU, row-major, dtype matching ``dtype``):
      W_q [d_model, H*d_q], subkeys [H, 2, n_sub, d_q/2], values [n_sub^2, d_value],
      W1 [d_model, d_value] and W2 [d_value, d_model] when ``memory_plus``.
    ``values`` is borrowed: keep it alive and unchanged while this object is used.  It may
    live in pinned host memory (a host-resident table, read over the host link); the
    workspace is allocated on W_q's device.
    """

    def __init__(self, *, d_model, n_heads, d_query, n_sub, k, d_value, dtype, qk_norm, memory_plus, max_tokens,
                 W_q, subkeys, values, W1=None, W2=None, norm_eps=1e-6, stream=None):
        import torch

        self.cfg = make_config(d_model, n_heads, d_query, n_sub, k, d_value, dtype, qk_norm, memory_plus, max_tokens,
                               norm_eps)
        self.dtype = {"f32": torch.float32, "bf16": torch.bfloat16}.get(dtype) or (
            torch.bfloat16 if dtype == PKM_BF16 else torch.float32)
        # the C ABI takes bare pointers: shapes, types and layouts are checked here, so that no
        # kernel reads past the end of a tensor
        want = [("W_q", W_q, (d_model, n_heads * d_query), False),
                ("subkeys", subkeys, (n_heads, 2, n_sub, d_query // 2), False),
                ("values", values, (n_sub * n_sub, d_value), True)]
        if memory_plus:
            want += [("W1", W1, (d_model, d_value), False), ("W2", W2, (d_value, d_model), False)]
        for device in (False, True):  # every shape, type and layout first, then where they live
            for name, t, shape, host_ok in want:
                _check_tensor(name, t, shape, self.dtype, host_ok=host_ok, device=device)
        self.ws_bytes = pkm_workspace_size(self.cfg)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=W_q.device)
        self._keep = (W_q, subkeys, values, W1, W2)
        self.handle = pkm_create(self.cfg, W_q, subkeys, values, W1, W2, self.workspace, self.ws_bytes, stream)

    @property
    def out_width(self) -> int:
        return self.cfg.d_model if self.cfg.memory_plus else self.cfg.d_value

    def forward(self, x, out=None, idx_out=None, w_out=None, stream=None):
        import torch

        T = x.shape[0] if getattr(x, "dim", lambda: 0)() == 2 else -1
        _check_tensor("x", x, (T, self.cfg.d_model), self.dtype)
        if out is None:
            out = torch.empty((T, self.out_width), dtype=x.dtype, device=x.device)
        _check_tensor("out", out, (T, self.out_width), self.dtype)
        sel = (T, self.cfg.n_heads, self.cfg.k)
        if idx_out is not None:
            _check_tensor("idx_out", idx_out, sel, torch.int32)
        if w_out is not None:
            _check_tensor("w_out", w_out, sel, torch.float32)
        pkm_forward(self.handle, x, T, out, idx_out, w_out, stream)
        return out

    def close(self):
        if getattr(self, "handle", None):
            pkm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
