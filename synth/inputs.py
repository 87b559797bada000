"""Host-side seeded generators (NumPy).

Every tensor is drawn from its own stream ``numpy.random.default_rng([seed, tid])``
with the tensor ids below, as float64 normals times a standard deviation,
rounded to float32 and, for bf16 workloads, rounded again to bf16 with
round-to-nearest-even.  bf16 tensors are returned as ``uint16`` bit patterns so
that the oracle and the GPU see the same stored bytes.

Standard deviations (input recipe): x ~ N(0, 1); W_q ~ N(0, 1/d_model);
sub-keys ~ N(0, 1/d_h) (std = 1/sqrt(fan-in)); W1, W2 ~ N(0, 0.02^2);
values ~ N(0, 0.02^2) through the row-addressable generator below.

The value table is row-addressable so that a 64-128 GiB table can be filled on
the GPU and any of its rows regenerated on the host:

    seed_V = splitmix64((seed << 8) | tid)       (tid = 6 for the value table)
    u      = splitmix64(seed_V XOR (row * d_v + col))
    S      = sum of the four 16-bit limbs of u          (Irwin-Hall, n = 4)
    v      = (S - 131070) * VALUE_SCALE                (IEEE float64)
    stored = float32(v), then bf16(float32(v)) for bf16 tables (both RNE)

splitmix64 is the mixing function of Steele, Lea and Flood, "Fast splittable
pseudorandom number generators" (OOPSLA 2014).  VALUE_SCALE = 0.02 / sd(S) with
sd(S) = sqrt(4 * (65536^2 - 1) / 12), so v has standard deviation 0.02 and is
bounded by about +-3.46 sd.
"""

from __future__ import annotations

import numpy as np

from .configs import Config

TID_X, TID_WQ, TID_KEYS, TID_W1, TID_W2, TID_V, TID_UIDX, TID_TOKENS, TID_HIDDEN = range(1, 10)
TID_ENGRAM, TID_MULT, TID_COMPRESS = 10, 11, 12

VALUE_SCALE = float.fromhex("0x1.1bc779ef9b324p-21")  # 0.02 / 37837.2272...
IRWIN_HALL_MEAN = 131070

_M64 = (1 << 64) - 1


def splitmix64_scalar(z: int) -> int:
    """splitmix64 output for state ``z`` (pure Python ints, for seeds and tests)."""
    z = (z + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def splitmix64(z: np.ndarray) -> np.ndarray:
    """Vectorised splitmix64 on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = z + np.uint64(0x9E3779B97F4A7C15)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def value_seed(seed: int, tid: int = TID_V) -> int:
    return splitmix64_scalar(((seed << 8) | tid) & _M64)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(v64: np.ndarray, dtype: str) -> np.ndarray:
    f32 = v64.astype(np.float32)
    return f32 if dtype == "f32" else f32_to_bf16_bits(f32)


def normal_tensor(seed: int, tid: int, shape, std: float, dtype: str) -> np.ndarray:
    rng = np.random.default_rng([seed, tid])
    return _store(rng.standard_normal(size=shape) * std, dtype)


def value_rows(seed: int, rows, d_v: int, dtype: str, tid: int = TID_V) -> np.ndarray:
    """Rows ``rows`` of the row-addressable table of tensor id ``tid`` (default: the
    value table), shape [len(rows), d_v] (float32 or bf16 bits)."""
    rows = np.asarray(rows, dtype=np.uint64).reshape(-1)
    sv = np.uint64(value_seed(seed, tid))
    ctr = rows[:, None] * np.uint64(d_v) + np.arange(d_v, dtype=np.uint64)[None, :]
    u = splitmix64(sv ^ ctr)
    m = np.uint64(0xFFFF)
    s = (u & m) + ((u >> np.uint64(16)) & m) + ((u >> np.uint64(32)) & m) + (u >> np.uint64(48))
    v64 = (s.astype(np.int64) - IRWIN_HALL_MEAN).astype(np.float64) * VALUE_SCALE
    return _store(v64, dtype)


def value_table(seed: int, n_rows: int, d_v: int, dtype: str, chunk: int = 1 << 14, tid: int = TID_V) -> np.ndarray:
    """The whole table (small tables only)."""
    out = np.empty((n_rows, d_v), dtype=np.float32 if dtype == "f32" else np.uint16)
    for r0 in range(0, n_rows, chunk):
        r1 = min(n_rows, r0 + chunk)
        out[r0:r1] = value_rows(seed, np.arange(r0, r1), d_v, dtype, tid)
    return out


def make_inputs(cfg: Config, seed: int = 0, T: int | None = None) -> dict:
    """Dense inputs of one workload: x, W_q, subkeys, and W1, W2 when the gate is on.

    Layouts (row-major): x [T, d_model]; W_q [d_model, H*d_q] (head h owns columns
    h*d_q .. h*d_q + d_q - 1); subkeys [H, 2, n_sub, d_h] (index 0 scores the
    first half of the query, 1 the second); W1 [d_model, d_v]; W2 [d_v, d_model].
    ``T`` overrides the token count (x is drawn for the full count and cut, so a
    shorter T gives a prefix of the same tokens).
    """
    t_full = cfg.T
    T = t_full if T is None else T
    d = {
        "x": normal_tensor(seed, TID_X, (max(T, t_full), cfg.d_model), 1.0, cfg.dtype)[:T],
        "W_q": normal_tensor(seed, TID_WQ, (cfg.d_model, cfg.H * cfg.d_q), cfg.d_model ** -0.5, cfg.dtype),
        "subkeys": normal_tensor(seed, TID_KEYS, (cfg.H, 2, cfg.n_sub, cfg.d_h), cfg.d_h ** -0.5, cfg.dtype),
    }
    if cfg.memory_plus:
        d["W1"] = normal_tensor(seed, TID_W1, (cfg.d_model, cfg.d_v), 0.02, cfg.dtype)
        d["W2"] = normal_tensor(seed, TID_W2, (cfg.d_v, cfg.d_model), 0.02, cfg.dtype)
    d["x"] = np.ascontiguousarray(d["x"])
    return d


def uniform_bags(seed: int, n_bags: int, bag: int, n_rows: int):
    """Uniform i.i.d. row indices and positive weights normalised per bag (gather microbench)."""
    rng = np.random.default_rng([seed, TID_UIDX])
    idx = rng.integers(0, n_rows, size=(n_bags, bag), dtype=np.int64).astype(np.int32)
    w = rng.random(size=(n_bags, bag)) + 0.5
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx, w


# ---- hashed n-gram lookup (Engram) inputs ---------------------------------------------

def zipf_tokens(seed: int, T: int, vocab: int, s: float) -> np.ndarray:
    """T token ids: rank r in 1..vocab drawn with probability proportional to r^-s
    (a Zipf law truncated at the vocabulary), id = r - 1; int32."""
    rng = np.random.default_rng([seed, TID_TOKENS])
    p = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    u = rng.random(T)
    return np.minimum(np.searchsorted(cdf, u, side="right"), vocab - 1).astype(np.int32)


def hidden_states(seed: int, T: int, d: int, dtype: str) -> np.ndarray:
    """h ~ N(0, 1), [T, d]."""
    return normal_tensor(seed, TID_HIDDEN, (T, d), 1.0, dtype)


def engram_multipliers(seed: int, min_order: int, n_orders: int, heads: int) -> np.ndarray:
    """Odd 64-bit multipliers m[o, k] of the hash of order n = min_order + o, head k:
    splitmix64(base XOR (n << 8 | k)) with the low bit set, base = splitmix64((seed << 8) | 11)."""
    base = splitmix64_scalar(((seed << 8) | TID_MULT) & _M64)
    m = np.empty((n_orders, heads), dtype=np.uint64)
    for o in range(n_orders):
        for k in range(heads):
            m[o, k] = splitmix64_scalar(base ^ (((min_order + o) << 8) | k)) | 1
    return m


def compress_map(seed: int, vocab: int, n_concepts: int) -> np.ndarray:
    """A vocabulary map onto n_concepts ids (uniform, many-to-one), int32 [vocab]."""
    rng = np.random.default_rng([seed, TID_COMPRESS])
    return rng.integers(0, n_concepts, size=vocab, dtype=np.int64).astype(np.int32)


def engram_table_rows(seed: int, rows, head_dim: int, dtype: str) -> np.ndarray:
    """Rows of the stacked Engram tables (tensor id 10), N(0, 0.02^2) like the value table."""
    return value_rows(seed, rows, head_dim, dtype, tid=TID_ENGRAM)


def make_engram_inputs(cfg, seed: int = 0, T: int | None = None) -> dict:
    """ids [T] int32, h [T, d], mult [n_orders, heads] uint64 and, with a vocabulary map,
    compress [vocab] int32.  ``T`` takes a prefix of the full workload's tokens."""
    T = cfg.T if T is None else T
    full = max(T, cfg.T)
    d = {
        "ids": zipf_tokens(seed, full, cfg.vocab, cfg.zipf_s)[:T].copy(),
        "h": np.ascontiguousarray(hidden_states(seed, full, cfg.d, cfg.dtype)[:T]),
        "mult": engram_multipliers(seed, cfg.min_order, cfg.n_orders, cfg.heads),
        "compress": compress_map(seed, cfg.vocab, cfg.n_concepts) if cfg.n_concepts else None,
    }
    return d


# ---- Memory Attention token-memory inputs ------------------------------------------

TID_MA_TABLE, TID_MA_KEYS, TID_MA_GAIN = 13, 14, 15


def make_ma_inputs(cfg, seed: int = 0, T: int | None = None) -> dict:
    """ids [T] int32 (Zipf), E [vocab, d_v] ~ N(0, 0.02^2) (stored dtype), K [T, d_v] ~ N(0, 1),
    gain [d_v] float32 ~ 1 + N(0, 0.1^2) (or None)."""
    T = cfg.T if T is None else T
    full = max(T, cfg.T)
    return {
        "ids": zipf_tokens(seed, full, cfg.vocab, cfg.zipf_s)[:T].copy(),
        "E": normal_tensor(seed, TID_MA_TABLE, (cfg.vocab, cfg.d_v), 0.02, cfg.dtype),
        "K": np.ascontiguousarray(normal_tensor(seed, TID_MA_KEYS, (full, cfg.d_v), 1.0, cfg.dtype)[:T]),
        "gain": ((1.0 + 0.1 * np.random.default_rng([seed, TID_MA_GAIN]).standard_normal(cfg.d_v)).astype(np.float32)
                 if cfg.gain else None),
    }
