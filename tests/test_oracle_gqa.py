"""Pins of the grouped-query / unequal-length oracle: float64 torch SDPA on
KV heads expanded to the query heads with an explicit bottom-right mask (a
library routine), reduction to the square single-head-group definition,
and closed forms of the alignment."""

import numpy as np
import pytest
import torch

from oracle import attention_gqa_ref, attention_ref

RNG = np.random.default_rng(30)


def _sdpa(q, k, v, causal, scale):
    G = q.shape[1] // k.shape[1]
    kk = torch.tensor(k).repeat_interleave(G, dim=1)
    vv = torch.tensor(v).repeat_interleave(G, dim=1)
    Nq, Nk = q.shape[2], k.shape[2]
    mask = None
    if causal:
        mask = torch.arange(Nk)[None, :] <= torch.arange(Nq)[:, None] + (Nk - Nq)
    return torch.nn.functional.scaled_dot_product_attention(torch.tensor(q), kk, vv, attn_mask=mask,
                                                            scale=scale).numpy()


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (6, 1), (8, 2)])
@pytest.mark.parametrize("Nq,Nk", [(1, 77), (5, 40), (40, 40), (33, 130)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(Hq, Hkv, Nq, Nk, causal):
    d = 16
    q = RNG.standard_normal((2, Hq, Nq, d))
    k, v = (RNG.standard_normal((2, Hkv, Nk, d)) for _ in range(2))
    o, lse = attention_gqa_ref(q, k, v, causal=causal, scale=0.25, row_block=16)
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal, float(np.float32(0.25))), rtol=1e-10, atol=1e-12)
    assert np.all(np.isfinite(lse))


@pytest.mark.parametrize("causal", [False, True])
def test_square_one_group_is_the_definition(causal):
    q, k, v = (RNG.standard_normal((1, 3, 50, 8)) for _ in range(3))
    o, lse = attention_gqa_ref(q, k, v, causal=causal)
    o2, lse2 = attention_ref(q, k, v, causal=causal)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)


def test_alignment_closed_forms():
    Nk, d = 9, 4
    q = RNG.standard_normal((1, 1, 3, d))
    k, v = (RNG.standard_normal((1, 1, Nk, d)) for _ in range(2))
    # one query (decode) sees every key: causal equals non-causal
    o1, l1 = attention_gqa_ref(q[:, :, :1], k, v, causal=True)
    o2, l2 = attention_gqa_ref(q[:, :, :1], k, v, causal=False)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    # with Q = 0 the last query sees all Nk keys: the mean of V and ln Nk
    z = np.zeros((1, 1, 3, d))
    o, lse = attention_gqa_ref(z, k, v, causal=True)
    np.testing.assert_allclose(o[0, 0, 2], v[0, 0].mean(axis=0), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log([Nk - 2, Nk - 1, Nk]), atol=1e-14)


def test_rows_that_see_no_key():
    # Nq > Nk, causal: the first Nq - Nk queries see nothing -> O = 0, lse = -inf
    q = RNG.standard_normal((1, 2, 10, 4))
    k, v = (RNG.standard_normal((1, 1, 4, 4)) for _ in range(2))
    o, lse = attention_gqa_ref(q, k, v, causal=True)
    assert np.all(o[:, :, :6] == 0) and np.all(np.isneginf(lse[:, :, :6]))
    assert np.all(np.isfinite(lse[:, :, 6:]))
    # query 6 is position 0 of the keys: it sees key 0 only
    np.testing.assert_allclose(o[0, :, 6], np.repeat(v[0, 0, :1], 2, axis=0), atol=1e-14)
