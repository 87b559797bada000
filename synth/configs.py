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


@dataclass(frozen=True)
class EngramConfig:
    """Hashed n-gram lookup (Engram review: multi-head hashing into per-(n, head)
    tables, eq. 1; context-aware gate, eq. 2)."""
    name: str
    T: int             # tokens
    seq_len: int       # tokens per sequence (n-grams never cross a sequence start)
    vocab: int         # token ids are in [0, vocab)
    zipf_s: float      # token ranks follow a truncated Zipf law P(r) ~ r^-s, id = r - 1
    min_order: int     # smallest n
    n_orders: int      # orders min_order .. min_order + n_orders - 1
    heads: int         # hash heads per order
    head_dim: int      # embedding width of one head; d = heads * head_dim
    table_rows: int    # rows of every table E_{n,k} (a prime)
    dtype: str         # "f32" or "bf16": tables, hidden states and output
    residual: bool = False   # out = h + alpha * e instead of alpha * e
    n_concepts: int = 0      # > 0: token ids first pass through a vocabulary map onto this many ids
    norm_eps: float = 1e-6

    @property
    def d(self) -> int:
        return self.heads * self.head_dim

    @property
    def n_tables(self) -> int:
        return self.n_orders * self.heads

    @property
    def total_rows(self) -> int:
        return self.n_tables * self.table_rows

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "EngramConfig":
        return replace(self, **kw)


ENGRAM_CONFIGS = {
    # 16,384 Zipf(1.1) token ids over a 128,000 vocabulary, 2- and 3-grams, 8 heads per
    # order, 16 tables of 2,097,143 (prime) rows x 128 bf16 (8.0 GiB), d = 1024
    "engram_zipf_2m_bf16": EngramConfig("engram_zipf_2m_bf16", T=16384, seq_len=16384, vocab=128000, zipf_s=1.1,
                                        min_order=2, n_orders=2, heads=8, head_dim=128, table_rows=2097143,
                                        dtype="bf16"),
    # small fp32 case: three sequences of 200 tokens, 4 heads of width 32, 1,009-row tables
    "engram_tiny_f32": EngramConfig("engram_tiny_f32", T=600, seq_len=200, vocab=500, zipf_s=1.1, min_order=2,
                                    n_orders=2, heads=4, head_dim=32, table_rows=1009, dtype="f32"),
    # vocabulary map onto 3,000 concept ids, orders 2..4, residual output
    "engram_compress_bf16": EngramConfig("engram_compress_bf16", T=1000, seq_len=250, vocab=5000, zipf_s=1.1,
                                         min_order=2, n_orders=3, heads=8, head_dim=64, table_rows=10007,
                                         dtype="bf16", residual=True, n_concepts=3000),
}

ENGRAM_HEADLINE = "engram_zipf_2m_bf16"


@dataclass(frozen=True)
class MemoryAttentionConfig:
    """Token-memory values of Memory Attention: a per-layer table E [vocab, d_v] read by
    token id, normalised per key/value head and added to the keys (V = K + Norm(E)[s])."""
    name: str
    T: int            # tokens (batch x sequence)
    vocab: int        # rows of the table
    d_v: int          # value width = n_heads * head_dim
    n_heads: int      # key/value heads; the norm runs over each head's slice of a row
    dtype: str        # "f32" or "bf16": E, K, V
    zipf_s: float = 1.1   # token ids follow a truncated Zipf law
    gain: bool = True     # a per-channel RMSNorm gain (fp32, [d_v])
    norm_eps: float = 1e-6

    @property
    def head_dim(self) -> int:
        return self.d_v // self.n_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "MemoryAttentionConfig":
        return replace(self, **kw)


MA_CONFIGS = {
    # the inference setting the page measures: hidden 2,048 with 32 key/value heads,
    # a 32,000-token vocabulary, batch 8 x 2,048 prefill tokens
    "ma_values_32k_bf16": MemoryAttentionConfig("ma_values_32k_bf16", T=16384, vocab=32000, d_v=2048, n_heads=32,
                                                dtype="bf16"),
    "ma_tiny_f32": MemoryAttentionConfig("ma_tiny_f32", T=300, vocab=700, d_v=96, n_heads=3, dtype="f32"),
}

MA_HEADLINE = "ma_values_32k_bf16"
