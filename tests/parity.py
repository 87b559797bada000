"""Comparison rules between the GPU path and the oracle (CPU side, used by GPU tests).

Index lists: at every position either the GPU's index equals the oracle's, or the
oracle's own float64 score of the GPU's choice lies within
tau = 1e-4 * max(1, |oracle score at that position|) of the oracle's score there
(a near-tie the rounding of the GPU arithmetic may order differently).  A GPU list
never holds an index twice.

Outputs: per token row, max|gpu - ref| <= tol * max|ref|, with tol = 1e-4 for fp32
and 2e-2 for bf16 storage.  The reference for a row is the oracle evaluated on the
GPU's own index set (its weights recomputed from the oracle's scores of those
indices), so rows with excused near-ties are checked too.
"""

from __future__ import annotations

import numpy as np

from oracle import pkm as O

TAU = 1e-4
TOL = {"f32": 1e-4, "bf16": 2e-2}


def check_lists(gpu_idx: np.ndarray, ora_idx: np.ndarray, ora_sc: np.ndarray, gpu_choice_score: np.ndarray,
                what: str) -> int:
    """All arrays [R, k]; gpu_choice_score = oracle float64 score of each GPU index. Returns #excused."""
    gpu_idx = gpu_idx.reshape(-1, gpu_idx.shape[-1])
    ora_idx = ora_idx.reshape(gpu_idx.shape)
    ora_sc = ora_sc.reshape(gpu_idx.shape)
    gs = gpu_choice_score.reshape(gpu_idx.shape)
    srt = np.sort(gpu_idx, axis=1)
    dup = (srt[:, 1:] == srt[:, :-1]).any(axis=1)
    assert not dup.any(), f"{what}: duplicate indices in {int(dup.sum())} GPU lists"
    diff = gpu_idx != ora_idx
    tau = TAU * np.maximum(1.0, np.abs(ora_sc))
    bad = diff & (np.abs(gs - ora_sc) > tau)
    if bad.any():
        r, j = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} positions differ beyond the near-tie margin; first at row {r} pos {j}: "
            f"gpu {gpu_idx[r, j]} (oracle score {gs[r, j]!r}) vs oracle {ora_idx[r, j]} ({ora_sc[r, j]!r})")
    return int(diff.sum())


def half_choice_scores(q1, q2, K1, K2, half_idx):
    """Oracle score of every index in a [T, H, 2, k] list of per-half sub-key choices."""
    T, H, _, k = half_idx.shape
    out = np.empty(half_idx.shape, dtype=np.float64)
    for c, (q, K) in enumerate(((q1, K1), (q2, K2))):
        for h in range(H):
            keys = K[h][half_idx[:, h, c, :]]            # [T, k, d_h]
            out[:, h, c, :] = np.einsum("tkd,td->tk", keys, q[:, h, :])
    return out


def cell_choice_scores(q1, q2, K1, K2, flat_idx):
    """Oracle score of every flat index in a [T, H, k] list."""
    n = K1.shape[1]
    a, b = np.divmod(flat_idx.astype(np.int64), n)
    T, H, k = flat_idx.shape
    out = np.empty(flat_idx.shape, dtype=np.float64)
    for h in range(H):
        out[:, h, :] = (np.einsum("tkd,td->tk", K1[h][a[:, h, :]], q1[:, h, :]) +
                        np.einsum("tkd,td->tk", K2[h][b[:, h, :]], q2[:, h, :]))
    return out


def check_rows(gpu: np.ndarray, ref: np.ndarray, tol: float, what: str) -> float:
    gpu = gpu.astype(np.float64).reshape(gpu.shape[0], -1)
    ref = ref.reshape(gpu.shape)
    err = np.abs(gpu - ref).max(axis=1)
    scale = np.abs(ref).max(axis=1)
    rel = err / np.maximum(scale, 1e-300)
    worst = int(np.argmax(rel))
    assert (err <= tol * scale).all(), (
        f"{what}: {int((err > tol * scale).sum())} rows off; worst row {worst}: rel err {rel[worst]:.3e} > {tol:.1e}")
    return float(rel.max())


def reference_on_gpu_choice(q1, q2, K1, K2, gpu_idx, rows_of):
    """Oracle y evaluated on the GPU's index sets: softmax of the oracle's scores of those indices."""
    sc = cell_choice_scores(q1, q2, K1, K2, gpu_idx)
    w = O.softmax(sc)
    return O.weighted_bag(rows_of, gpu_idx.astype(np.int64), w), w


def max_ulp_bf16(a_bits: np.ndarray, b_bits: np.ndarray) -> int:
    """Largest distance in bf16 units in the last place between two arrays of bf16 patterns."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x & 0x7FFF)
    return int(np.abs(ordered(a_bits) - ordered(b_bits)).max()) if a_bits.size else 0


def check_bf16_rounded(gpu_bits: np.ndarray, ref: np.ndarray, abs_slack: float, what: str, ulps: float = 1.0) -> None:
    """Each GPU bf16 value lies within `ulps` bf16 ulps of the float64 reference, after allowing
    `abs_slack` for the fp32 accumulation that produced the value before rounding
    (a dot product over d_model terms can cancel, so near-zero outputs carry an
    absolute, not a relative, error).  One ulp covers a single rounding of the result."""
    g = O.bf16_bits_to_f64(gpu_bits).reshape(ref.shape)
    mag = np.maximum(np.abs(ref), 1e-30)
    ulp = 2.0 ** (np.floor(np.log2(mag)) - 7)
    excess = np.abs(g - ref) - (ulps * ulp + abs_slack)
    assert (excess <= 0).all(), (f"{what}: {int((excess > 0).sum())} values beyond {ulps:g} bf16 ulp + {abs_slack:g}; "
                                 f"worst excess {excess.max():.3e}")
