"""Attention over a batch of variable-length sequences packed end to end.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

The FA3 explainer lists variable-length batches among the shapes a kernel is
dispatched on (P1 section "安装了包，为什么可能没有用上 FA3") and asks tests to
cover very short and empty valid ranges in them (section "正确性验证要覆盖异步
边界"); it fixes no layout.  Readings taken:

* Packing: sequence b owns query rows cu_q[b] .. cu_q[b+1] - 1 and key rows
  cu_k[b] .. cu_k[b+1] - 1 of token-major tensors q ``[total_q, Hq, d]``,
  k, v ``[total_k, Hkv, d]`` (the layout of the usual packed attention
  interface); o is ``[total_q, Hq, d]`` and lse ``[Hq, total_q]``.
* Each sequence is an independent attention problem with the grouped-head
  map and bottom-right causal alignment of :mod:`oracle.gqa`; queries never
  see another sequence's keys.
* A query row that sees no key (a sequence with no keys, or causal rows
  before the first visible key) has O = 0 and lse = -inf.
"""

from __future__ import annotations

import numpy as np

from .attention import to_f64
from .gqa import attention_gqa_ref

__all__ = ["attention_varlen_ref"]


def attention_varlen_ref(q, k, v, cu_q, cu_k, causal: bool = False, scale=None):
    """O ``[total_q, Hq, d]`` and lse ``[Hq, total_q]`` (float64) of the packed batch."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    cu_q = [int(x) for x in np.asarray(cu_q)]
    cu_k = [int(x) for x in np.asarray(cu_k)]
    total_q, Hq, d = q.shape
    o = np.zeros((total_q, Hq, v.shape[2]))
    lse = np.full((Hq, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if q1 <= q0 or k1 <= k0:
            continue  # no queries, or no keys: O = 0, lse = -inf
        qb = q[q0:q1].transpose(1, 0, 2)[None]
        kb = k[k0:k1].transpose(1, 0, 2)[None]
        vb = v[k0:k1].transpose(1, 0, 2)[None]
        ob, lb = attention_gqa_ref(qb, kb, vb, causal=causal, scale=scale)
        o[q0:q1] = ob[0].transpose(1, 0, 2)
        lse[:, q0:q1] = lb[0]
    return o, lse
