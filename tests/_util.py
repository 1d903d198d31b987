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


def check_rows(o, lse, o_ref, lse_ref, label, gate=(1e-2, 2e-3, 1e-2), lse_gate=1e-3):
    """Bf16-path gates on the rows that see at least one key (max-abs, RMSE,
    relative RMSE of O; max-abs of lse), and O = 0, lse = -inf exactly on
    the rows that see none (lse_ref = -inf)."""
    o, lse = np.asarray(o), np.asarray(lse)
    seen = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), seen), label
    assert np.all(o[~seen] == 0) and np.all(np.isneginf(lse[~seen])), label
    assert np.isfinite(o).all(), label
    e = errors(o[seen], o_ref[seen])
    el = float(np.abs(lse[seen].astype(np.float64) - lse_ref[seen]).max()) if seen.any() else 0.0
    print(f"{label}: max_abs={e['max_abs']:.3e} rmse={e['rmse']:.3e} rel_rmse={e['rel_rmse']:.3e} lse={el:.3e}")
    assert e["max_abs"] <= gate[0] and e["rmse"] <= gate[1] and e["rel_rmse"] <= gate[2], (label, e)
    assert el <= lse_gate, (label, el)
