"""Device-side helpers shared by the GPU tests, smoke() and bench.py.

Moves the seeded synthetic inputs to the GPU, fills the value table there with the
device generator, and builds a ProductKeyMemory over them.  No forward arithmetic
happens here.
"""

from __future__ import annotations

import numpy as np
import torch

from synth import inputs as S

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a.astype(np.float32, copy=False)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def make_value_table(cfg, seed: int = 0) -> torch.Tensor:
    from synth import device as SD
    v = torch.empty((cfg.N, cfg.d_v), dtype=TORCH_DT[cfg.dtype], device="cuda")
    SD.fill_values(v, seed)
    return v


class Workload:
    """Inputs of one workload on the GPU plus a handle over them."""

    def __init__(self, cfg, seed: int = 0, T: int | None = None, max_tokens: int | None = None,
                 values: torch.Tensor | None = None, host_inputs: dict | None = None, value_seed: int | None = None):
        """``values`` (with the ``value_seed`` it was filled from) shares one value table
        between several workloads (a shared memory pool)."""
        import sparse_key_value_amd as P

        self.cfg, self.seed = cfg, seed
        self.value_seed = seed if value_seed is None else value_seed
        self.T = cfg.T if T is None else T
        self.inp = host_inputs if host_inputs is not None else S.make_inputs(cfg, seed, T=self.T)
        self.dev = {k: to_dev(v, cfg.dtype) for k, v in self.inp.items()}
        self.values = values if values is not None else make_value_table(cfg, self.value_seed)
        self.pkm = P.ProductKeyMemory(
            d_model=cfg.d_model, n_heads=cfg.H, d_query=cfg.d_q, n_sub=cfg.n_sub, k=cfg.k, d_value=cfg.d_v,
            dtype=cfg.dtype, qk_norm=cfg.qk_norm, memory_plus=cfg.memory_plus,
            max_tokens=max_tokens or max(1, self.T), norm_eps=cfg.norm_eps, W_q=self.dev["W_q"],
            subkeys=self.dev["subkeys"], values=self.values, W1=self.dev.get("W1"), W2=self.dev.get("W2"))

    def host_rows(self, rows) -> np.ndarray:
        """Stored value rows as generated on the host (float32 or bf16 bits)."""
        return S.value_rows(self.value_seed, rows, self.cfg.d_v, self.cfg.dtype)

    def forward_debug(self, x: torch.Tensor | None = None):
        import sparse_key_value_amd as P

        cfg = self.cfg
        x = self.dev["x"] if x is None else x
        T = x.shape[0]
        dt = TORCH_DT[cfg.dtype]
        o = {
            "qhat": torch.empty((T, cfg.H, 2, cfg.d_h), dtype=dt, device="cuda"),
            "half_idx": torch.empty((T, cfg.H, 2, cfg.k), dtype=torch.int32, device="cuda"),
            "half_score": torch.empty((T, cfg.H, 2, cfg.k), dtype=torch.float32, device="cuda"),
            "idx": torch.empty((T, cfg.H, cfg.k), dtype=torch.int32, device="cuda"),
            "score": torch.empty((T, cfg.H, cfg.k), dtype=torch.float32, device="cuda"),
            "w": torch.empty((T, cfg.H, cfg.k), dtype=torch.float32, device="cuda"),
            "y": torch.empty((T, cfg.d_v), dtype=torch.float32, device="cuda"),
        }
        out = torch.empty((T, cfg.d_out), dtype=dt, device="cuda")
        P.pkm_forward_debug(self.pkm.handle, x, T, out, o)
        torch.cuda.synchronize()
        o["out"] = out
        return o

    def close(self):
        self.pkm.close()
