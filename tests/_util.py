"""Shared helpers of the GPU parity tests (no attention arithmetic here)."""

from __future__ import annotations

import numpy as np


def errors(got, ref):
    """max-abs, RMSE, relative RMSE (RMSE / rms(ref)) and cosine of two arrays."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    rmse = float(np.sqrt(np.mean(d * d))) if d.size else 0.0
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    nn = float(np.sqrt((got * got).sum() * (ref * ref).sum())) if ref.size else 0.0
    if nn > 0:
        cos = float((got * ref).sum() / nn)
    else:  # an all-zero side: agreement only if both are zero
        cos = 1.0 if rmse == 0.0 else 0.0
    return {
        "max_abs": float(np.abs(d).max()) if d.size else 0.0,
        "rmse": rmse,
        "rel_rmse": rmse / rms if rms > 0 else (0.0 if rmse == 0.0 else float("inf")),
        "cos": cos,
    }


def sample_rows(N: int, tile: int = 128, extra: int = 16, seed: int = 0):
    """Query rows that cover the first/last rows, every tile edge near the
    start and the end, and a few random rows in between."""
    rows = {0, 1, N - 1, N - 2}
    for t in (1, 2, 3):
        for e in (t * tile - 1, t * tile, t * tile + 1, N - t * tile, N - t * tile - 1):
            rows.add(e)
    rng = np.random.default_rng(seed)
    rows.update(int(r) for r in rng.integers(0, N, size=extra))
    return np.array(sorted(r for r in rows if 0 <= r < N), dtype=np.int64)
