"""Plain CPU fp64 attention: the definition and the tiled online recurrence.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Both functions take ``q, k, v`` of shape ``[B, H, N, d]`` (``v`` may have its
own last dimension), as NumPy arrays or CPU torch tensors of any float dtype.
They are upcast to float64 before any arithmetic, so a caller that hands in
the exact bf16 tensors the GPU received gets the exact real-valued problem.

``scale`` is the softmax scale as the library receives it, a float32; both
functions use ``float64(float32(scale))`` so that the GPU and the oracle see
the same constant.  When it is omitted it is ``1/sqrt(d)`` (P2 section 一.1,
where the scaling factor of scaled dot-product attention is 1/sqrt(d_k)).

Causal convention: query row ``i`` may attend to key ``j`` iff ``j <= i`` (the
lower triangle including the diagonal, P1 section "为什么 Causal Shape 可能更难调度";
queries and keys have the same length here, so there is no alignment choice).

The logsumexp output is the natural log of the row's sum of exp(S_ij) over
the keys it may attend to; the pages never define it, and this is the plain
reading.
"""

from __future__ import annotations

import numpy as np

__all__ = ["attention_ref", "online_ref", "to_f64", "scale_f64"]


def to_f64(x) -> np.ndarray:
    """Upcast a NumPy array or a CPU torch tensor (bf16 included) to float64."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64, copy=False)
    # torch tensors: go through float32, which holds every bf16 value exactly
    import torch

    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def scale_f64(scale, d: int) -> float:
    """The softmax scale as the GPU sees it: a float32, widened to float64."""
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    return float(np.float32(scale))


def attention_ref(q, k, v, causal: bool = False, scale=None, rows=None, row_block: int = 1024):
    """Scaled dot-product attention straight from its definition.

    O = softmax(scale * Q K^T) V, row by row, with S materialised in full for
    every query row computed (P2 section 一.1 defines the operation; P1
    section "FA3 没有改变什么" states the fused kernel still computes exact
    dense attention, so the definition is the oracle).

    Args:
      q, k, v: ``[B, H, N, d]`` / ``[B, H, Nk, d]`` / ``[B, H, Nk, dv]``.
      causal: mask keys ``j > i`` to -inf before the softmax.
      scale: float32 softmax scale (``None``: ``1/sqrt(d)``).
      rows: optional 1-D sequence of query indices; only those rows are
        computed (each output row depends on its own query alone).
      row_block: number of query rows whose full score rows are held at
        once; it only bounds memory, every row still sees every key.

    Returns:
      ``(o, lse)``: ``o`` float64 ``[B, H, R, dv]``, ``lse`` float64
      ``[B, H, R]`` (natural log), where R is N or ``len(rows)``.
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    sc = scale_f64(scale, d)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    o = np.empty((B, H, R, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    keys = np.arange(Nk)
    for b in range(B):
        for h in range(H):
            K = k[b, h]
            V = v[b, h]
            for r0 in range(0, R, row_block):
                idx = rows[r0:r0 + row_block]
                S = sc * (q[b, h, idx] @ K.T)  # [r, Nk], the full score rows
                if causal:
                    S = np.where(keys[None, :] > idx[:, None], -np.inf, S)
                m = S.max(axis=1)
                P = np.exp(S - m[:, None])
                l = P.sum(axis=1)
                o[b, h, r0:r0 + len(idx)] = (P @ V) / l[:, None]
                lse[b, h, r0:r0 + len(idx)] = m + np.log(l)
    return o, lse


def online_ref(q, k, v, causal: bool = False, scale=None, Bc: int = 64):
    """The tiled online-softmax recurrence over key blocks of ``Bc`` rows.

    State per query row: running max ``m``, running sum ``l`` and unnormalised
    output accumulator, initialised to (-inf, 0, 0) (P2 section 二.1 names the
    three states and their initial values; the update rules there and in P1
    section "Online Softmax 仍是精确合并的核心" were lost from the page text,
    so the standard rescaling recurrence is written here):

      m' = max(m, rowmax S_j)
      alpha = exp(m - m'),  P = exp(S_j - m')
      l = alpha * l + rowsum P,   acc = alpha * acc + P V_j,   m = m'

    and at the end O = acc / l, lse = m + ln l (normalisation deferred to the
    end, P1 "最后" in the same section).  A row whose running max is still
    -inf (every key so far masked) keeps alpha = 1 and P = 0.

    Every key block is visited; masked keys are -inf.  Returns float64
    ``(o, lse)`` like :func:`attention_ref`.
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    sc = scale_f64(scale, d)
    qi = np.arange(N)
    o = np.empty((B, H, N, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, v.shape[3]))
            for j0 in range(0, Nk, Bc):
                j1 = min(j0 + Bc, Nk)
                S = sc * (q[b, h] @ k[b, h, j0:j1].T)
                if causal:
                    S = np.where(np.arange(j0, j1)[None, :] > qi[:, None], -np.inf, S)
                m_new = np.maximum(m, S.max(axis=1))
                dead = np.isneginf(m_new)
                safe = np.where(dead, 0.0, m_new)
                alpha = np.where(dead, 1.0, np.exp(m - safe))
                P = np.where(dead[:, None], 0.0, np.exp(S - safe[:, None]))
                l = alpha * l + P.sum(axis=1)
                acc = alpha[:, None] * acc + P @ v[b, h, j0:j1]
                m = m_new
            o[b, h] = acc / l[:, None]
            lse[b, h] = m + np.log(l)
    return o, lse
