"""Plain CPU fp64 attention backward: the gradients of the forward's definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

The pages report backward speed-ups (P1 section "论文中的性能数字应该怎样理解")
and list dQ, dK, dV among the outputs a correctness suite must cover (P1
section "正确性验证要覆盖异步边界"), but give no formula: the backward is the
derivative of the forward the pages define (P2 section 一.1), written out.
For one (batch, head), with S = scale Q K^T (masked entries -inf),
P = softmax_rows(S), O = P V and an upstream gradient dO:

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij  (= sum_c dO_ic O_ic)
    dS = P * (dP - D)       (row-wise; masked entries have P = 0)
    dQ = scale dS K
    dK = scale dS^T Q

Inputs are upcast to float64 as in :mod:`oracle.attention` (the exact bf16
tensors given to the GPU are the exact real-valued problem); ``scale`` is
``float64(float32(scale))``; causal means key j <= query i.
"""

from __future__ import annotations

import numpy as np

from .attention import scale_f64, to_f64

__all__ = ["attention_bwd_ref", "attention_gqa_bwd_ref"]


def attention_bwd_ref(q, k, v, do, causal: bool = False, scale=None, row_block: int = 1024):
    """dQ, dK, dV of L = sum(O * dO) for O = attention(q, k, v).

    Args:
      q, k, v, do: ``[B, H, N, d]`` arrays or CPU tensors (any float dtype).
      causal: key j is visible to query i iff j <= i.
      scale: softmax scale (float32 semantics); default 1/sqrt(d).
      row_block: query rows per materialised block of S (memory cap only;
        dK and dV are summed over the blocks).

    Returns:
      ``(dq, dk, dv)`` float64 arrays shaped like ``q``, ``k``, ``v``.
    """
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    sc = scale_f64(scale, d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    kj = np.arange(Nk)
    for b in range(B):
        for h in range(H):
            Q, K, V, dO = q[b, h], k[b, h], v[b, h], do[b, h]
            for r0 in range(0, N, row_block):
                r1 = min(r0 + row_block, N)
                S = sc * (Q[r0:r1] @ K.T)
                if causal:
                    S = np.where(kj[None, :] > np.arange(r0, r1)[:, None], -np.inf, S)
                m = S.max(axis=1, keepdims=True)
                E = np.exp(S - m)
                P = E / E.sum(axis=1, keepdims=True)
                dOb = dO[r0:r1]
                dP = dOb @ V.T
                D = (P * dP).sum(axis=1, keepdims=True)
                dS = P * (dP - D)
                dq[b, h, r0:r1] = sc * (dS @ K)
                dk[b, h] += sc * (dS.T @ Q[r0:r1])
                dv[b, h] += P.T @ dOb
    return dq, dk, dv


def attention_gqa_bwd_ref(q, k, v, do, causal: bool = False, scale=None, row_block: int = 1024):
    """dQ, dK, dV with grouped/multi-query heads (equal query and key lengths).

    The forward of :mod:`oracle.gqa` lets query head h read KV head
    floor(h / G), G = Hq / Hkv: the same as giving every query head its own
    copy of that KV head.  By the chain rule, the gradient of a KV head is
    then the sum of the gradients of its G copies, each of which is the
    single-head gradient written out in :func:`attention_bwd_ref`.

    Args:
      q, do: ``[B, Hq, N, d]``; k, v: ``[B, Hkv, N, d]`` (Hq a multiple of Hkv).
      causal, scale, row_block: as :func:`attention_bwd_ref`.

    Returns:
      ``(dq, dk, dv)`` float64 arrays shaped like ``q``, ``k``, ``v``.
    """
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if k.shape[2] != N:
        raise ValueError("queries and keys must have the same length")
    G = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(Hq):
        hk = h // G
        gq, gk, gv = attention_bwd_ref(q[:, h:h + 1], k[:, hk:hk + 1], v[:, hk:hk + 1], do[:, h:h + 1],
                                       causal=causal, scale=scale, row_block=row_block)
        dq[:, h] = gq[:, 0]
        dk[:, hk] += gk[:, 0]
        dv[:, hk] += gv[:, 0]
    return dq, dk, dv
