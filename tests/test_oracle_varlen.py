"""Pins of the packed variable-length oracle: float64 torch SDPA per sequence
with an explicit bottom-right mask (a library routine), empty sequences and
sequences without keys (O = 0, lse = -inf), and independence from the other
sequences of the batch."""

import numpy as np
import pytest
import torch

from oracle import attention_varlen_ref

RNG = np.random.default_rng(40)


def _sdpa_seq(q, k, v, causal, scale):
    # q [Nq, Hq, d], k, v [Nk, Hkv, d] -> o [Nq, Hq, d]
    G = q.shape[1] // k.shape[1]
    qt = torch.tensor(q).transpose(0, 1)
    kt = torch.tensor(k).transpose(0, 1).repeat_interleave(G, dim=0)
    vt = torch.tensor(v).transpose(0, 1).repeat_interleave(G, dim=0)
    Nq, Nk = q.shape[0], k.shape[0]
    mask = None
    if causal:
        mask = torch.arange(Nk)[None, :] <= torch.arange(Nq)[:, None] + (Nk - Nq)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale).transpose(0, 1).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 1)])
def test_matches_sdpa_per_sequence(Hq, Hkv, causal):
    lq = [5, 1, 17, 9]
    lk = [5, 30, 17, 12]
    cu_q, cu_k = np.cumsum([0] + lq), np.cumsum([0] + lk)
    d = 8
    q = RNG.standard_normal((cu_q[-1], Hq, d))
    k, v = (RNG.standard_normal((cu_k[-1], Hkv, d)) for _ in range(2))
    o, lse = attention_varlen_ref(q, k, v, cu_q, cu_k, causal=causal, scale=0.4)
    for b in range(4):
        sl = slice(cu_q[b], cu_q[b + 1])
        ref = _sdpa_seq(q[sl], k[cu_k[b]:cu_k[b + 1]], v[cu_k[b]:cu_k[b + 1]], causal, float(np.float32(0.4)))
        np.testing.assert_allclose(o[sl], ref, rtol=1e-10, atol=1e-12)
    assert np.isfinite(lse).all()


def test_empty_sequences_and_sequences_without_keys():
    cu_q = np.array([0, 0, 4, 4, 7])   # sequence 0 and 2 have no queries
    cu_k = np.array([0, 3, 3, 5, 9])   # sequence 1 has no keys
    q = RNG.standard_normal((7, 2, 4))
    k, v = (RNG.standard_normal((9, 2, 4)) for _ in range(2))
    o, lse = attention_varlen_ref(q, k, v, cu_q, cu_k, causal=True)
    assert np.all(o[0:4] == 0) and np.all(np.isneginf(lse[:, 0:4]))
    # sequence 3: 3 queries against 4 keys, the last query sees all four
    z = np.zeros_like(q)
    o2, lse2 = attention_varlen_ref(z, k, v, cu_q, cu_k, causal=True)
    np.testing.assert_allclose(o2[6], v[5:9].mean(axis=0), atol=1e-14)
    np.testing.assert_allclose(lse2[:, 4:7], np.log([[2, 3, 4]] * 2), atol=1e-14)


def test_sequences_do_not_see_each_other():
    cu = np.array([0, 6, 10])
    q = RNG.standard_normal((10, 2, 4))
    k, v = (RNG.standard_normal((10, 2, 4)) for _ in range(2))
    o, lse = attention_varlen_ref(q, k, v, cu, cu)
    k2, v2 = k.copy(), v.copy()
    k2[6:] += 5.0  # change only sequence 1's keys and values
    v2[6:] -= 3.0
    o2, lse2 = attention_varlen_ref(q, k2, v2, cu, cu)
    np.testing.assert_array_equal(o[:6], o2[:6])
    np.testing.assert_array_equal(lse[:, :6], lse2[:, :6])
