"""Grouped-query attention and unequal query/key lengths, from the definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

The pages name grouped/multi-query attention (few KV heads shared by many
query heads) and queries shorter than keys (decode, prefill against a cache)
among the shapes an attention kernel meets, and list "Q/K 不同长度" among the
cases a correctness suite must cover (P1 sections "为什么 Causal Shape 可能更难
调度" and "正确性验证要覆盖异步边界"), but fix neither the head map nor the
causal alignment.  Readings taken:

* Head map: query head h reads KV head floor(h / G), G = Hq / Hkv (each KV
  head serves G consecutive query heads; Hkv = 1 is multi-query attention).
* Causal alignment, bottom-right: with Nq queries and Nk keys, query i is
  the (Nk - Nq + i)-th position and sees keys j <= i + Nk - Nq.  A single
  query (decode) then sees every key, and Nq = Nk is the square case of
  :mod:`oracle.attention`.
* A query row that sees no key at all (only when Nq > Nk) has no softmax;
  its output row is 0 and its logsumexp -inf (the empty sum).
"""

from __future__ import annotations

import numpy as np

from .attention import scale_f64, to_f64

__all__ = ["attention_gqa_ref"]


def attention_gqa_ref(q, k, v, causal: bool = False, scale=None, row_block: int = 1024):
    """O, lse for q ``[B, Hq, Nq, d]`` against k, v ``[B, Hkv, Nk, d]``.

    S = scale Q K^T of the mapped KV head, masked (bottom-right causal), P =
    softmax over the visible keys, O = P V; float64 outputs
    ``o [B, Hq, Nq, dv]`` and ``lse [B, Hq, Nq]`` (natural log).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    sc = scale_f64(scale, d)
    off = Nk - Nq
    o = np.zeros((B, Hq, Nq, v.shape[3]))
    lse = np.full((B, Hq, Nq), -np.inf)
    keys = np.arange(Nk)
    for b in range(B):
        for h in range(Hq):
            K, V = k[b, h // G], v[b, h // G]
            for r0 in range(0, Nq, row_block):
                idx = np.arange(r0, min(r0 + row_block, Nq))
                S = sc * (q[b, h, idx] @ K.T)
                if causal:
                    S = np.where(keys[None, :] > idx[:, None] + off, -np.inf, S)
                seen = ~np.all(np.isneginf(S), axis=1)
                if not seen.any():
                    continue
                Ss = S[seen]
                m = Ss.max(axis=1)
                P = np.exp(Ss - m[:, None])
                l = P.sum(axis=1)
                o[b, h, idx[seen]] = (P @ V) / l[:, None]
                lse[b, h, idx[seen]] = m + np.log(l)
    return o, lse
