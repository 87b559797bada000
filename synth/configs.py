"""Named workloads of the product-key memory forward.

Shapes follow the pages: product keys over about a million cells with about a
thousand half-keys per half ("Memory Layers at Scale" overview, section on how
product keys work), tables up to 64M keys ("Memory Layers at Scale" digest,
section on performance versus memory size) and roughly thirty values read per
token (overview, same section), hence k = 32.
"""

from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Config:
    name: str
    T: int            # tokens
    d_model: int      # width of x (and of the output when the Memory+ gate is on)
    H: int            # heads
    d_q: int          # per-head query width (even); each half is d_q // 2
    n_sub: int        # sub-keys per half; the table has n_sub ** 2 rows
    d_v: int          # value width
    k: int            # per-half top-k and final top-k
    dtype: str        # "f32" or "bf16": storage type of x, W_q, sub-keys, V, W1, W2, out
    qk_norm: bool     # RMSNorm on the query (before the split) and on each sub-key row
    memory_plus: bool  # out = (y * silu(x W1)) W2 instead of out = y
    norm_eps: float = 1e-6

    @property
    def d_h(self) -> int:
        return self.d_q // 2

    @property
    def N(self) -> int:
        return self.n_sub * self.n_sub

    @property
    def d_out(self) -> int:
        return self.d_model if self.memory_plus else self.d_v

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    # small fp32 case: 512 tokens, 65,536 values of width 256, no qk-norm, no gate
    "tiny_fp32_65k": Config("tiny_fp32_65k", T=512, d_model=256, H=1, d_q=128, n_sub=256,
                            d_v=256, k=32, dtype="f32", qk_norm=False, memory_plus=False),
    # 1M-key bf16 table of width 1024, 4 heads, qk-norm, no gate
    "pkm_1m_bf16": Config("pkm_1m_bf16", T=8192, d_model=1024, H=4, d_q=512, n_sub=1024,
                          d_v=1024, k=32, dtype="bf16", qk_norm=True, memory_plus=False),
    # Memory+ block: 16M keys x 2048 bf16 (64 GiB table), gate 2048 x 2048
    "memplus_16m_bf16": Config("memplus_16m_bf16", T=16384, d_model=2048, H=4, d_q=512,
                               n_sub=4096, d_v=2048, k=32, dtype="bf16", qk_norm=True,
                               memory_plus=True),
    # largest one-GPU table: 64M keys x 1024 bf16 (128 GiB), gate 1024 x 1024
    "memplus_64m_bf16": Config("memplus_64m_bf16", T=16384, d_model=1024, H=4, d_q=512,
                               n_sub=8192, d_v=1024, k=32, dtype="bf16", qk_norm=True,
                               memory_plus=True),
}

# the workload the throughput line is quoted on
HEADLINE = "memplus_16m_bf16"


def get_config(name: str) -> Config:
    return CONFIGS[name]
