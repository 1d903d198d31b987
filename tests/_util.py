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


def lazy_rescale_events(q, k, scale, tile, causal, lazy_log2=8.0, margin=0.02, group=32, off=0):
    """Count, for bf16 inputs q [.., Nq, d] and k [.., Nk, d], the (row, key
    tile) pairs at which the bf16 forward's lazy rescale fires with a finite
    running reference and moves that row's reference up by more than the
    threshold (times 1 + margin, so fp32 summation order cannot undo it).

    The forward keeps one exponent reference per query row and raises the
    references of a whole group of ``group`` consecutive rows (one wave)
    only when some row of the group sees a key tile whose row max exceeds
    its reference by more than lazy_log2 / (scale log2 e) raw score units.
    Query i sees keys j <= i + off when causal.  This is a prediction about
    the kernel's control flow, used to show that a test input exercises the
    rescale; it takes no part in any expected value."""
    qf = np.asarray(q, dtype=np.float64).reshape(-1, *np.shape(q)[-2:])
    kf = np.asarray(k, dtype=np.float64).reshape(-1, *np.shape(k)[-2:])
    thr = lazy_log2 / (scale * 1.4426950408889634)
    events = 0
    for qh, kh in zip(qf, kf):
        Nq, Nk = qh.shape[0], kh.shape[0]
        S = qh @ kh.T
        if causal:
            S = np.where(np.arange(Nk)[None, :] > np.arange(Nq)[:, None] + off, -np.inf, S)
        for r0 in range(0, Nq, group):
            Sg = S[r0:r0 + group]
            m = np.full(Sg.shape[0], -np.inf)
            for j0 in range(0, Nk, tile):
                mx = Sg[:, j0:j0 + tile].max(axis=1)
                grow = mx > m + thr
                if grow.any():
                    events += int(np.sum(np.isfinite(m) & (mx > m + thr * (1 + margin))))
                    m = np.maximum(m, mx)
    return events
