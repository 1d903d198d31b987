"""Pins of the backward oracle against facts that do not come from it:
torch autograd in float64 (a library routine), central finite differences,
and closed forms of the gradients."""

import numpy as np
import pytest
import torch

from oracle import attention_bwd_ref, attention_gqa_bwd_ref, attention_ref

RNG = np.random.default_rng(20)


def _autograd(q, k, v, do, causal, scale):
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    s = scale * t[0] @ t[1].transpose(-1, -2)
    if causal:
        n = q.shape[2]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ t[2]
    o.backward(torch.tensor(do))
    return [x.grad.numpy() for x in t]


@pytest.mark.parametrize("causal", [False, True])
def test_matches_float64_autograd(causal):
    B, H, N, d = 2, 2, 70, 16
    q, k, v, do = (RNG.standard_normal((B, H, N, d)) for _ in range(4))
    sc = 0.3
    got = attention_bwd_ref(q, k, v, do, causal=causal, scale=sc, row_block=32)
    ref = _autograd(q, k, v, do, causal, float(np.float32(sc)))
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_central_differences(causal):
    # L = sum(O * dO); dL/dx by central differences on a few entries of q, k, v
    B, H, N, d = 1, 1, 9, 4
    q, k, v, do = (RNG.standard_normal((B, H, N, d)) for _ in range(4))
    grads = attention_bwd_ref(q, k, v, do, causal=causal, scale=0.5)

    def loss(qq, kk, vv):
        o, _ = attention_ref(qq, kk, vv, causal=causal, scale=0.5)
        return float((o * do).sum())

    eps = 1e-6
    for which, g in enumerate(grads):
        for _ in range(6):
            i, c = int(RNG.integers(N)), int(RNG.integers(d))
            args = [q.copy(), k.copy(), v.copy()]
            args[which][0, 0, i, c] += eps
            up = loss(*args)
            args[which][0, 0, i, c] -= 2 * eps
            dn = loss(*args)
            assert abs((up - dn) / (2 * eps) - g[0, 0, i, c]) < 1e-7


@pytest.mark.parametrize("causal", [False, True])
def test_closed_forms(causal):
    B, H, N, d = 1, 2, 50, 8
    q, k, v, do = (RNG.standard_normal((B, H, N, d)) for _ in range(4))
    dq, dk, dv = attention_bwd_ref(q, k, v, do, causal=causal)
    # rows of P sum to 1: the dV rows sum to the dO rows' sum
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    # rows of dS sum to 0: the dK rows sum to zero
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    if causal:
        # query 0 sees key 0 only, so P_00 = 1 and its dS row vanishes
        np.testing.assert_allclose(dq[:, :, 0], 0.0, atol=1e-14)
    # no upstream gradient, no gradient
    z = attention_bwd_ref(q, k, v, np.zeros_like(do), causal=causal)
    for g in z:
        assert np.all(g == 0)


def test_q_zero_closed_form():
    # Q = 0 (non-causal): P is uniform 1/N, so dS_ij = (dO_i . (v_j - mean v)) / N
    # and dQ_i = scale / N sum_j (dO_i . (v_j - mean v)) k_j; dK = 0
    B, H, N, d = 1, 1, 30, 6
    k, v, do = (RNG.standard_normal((B, H, N, d)) for _ in range(3))
    q = np.zeros((B, H, N, d))
    sc = float(np.float32(0.7))
    dq, dk, dv = attention_bwd_ref(q, k, v, do, scale=0.7)
    vc = v[0, 0] - v[0, 0].mean(axis=0)
    expect = sc / N * (do[0, 0] @ vc.T) @ k[0, 0]
    np.testing.assert_allclose(dq[0, 0], expect, atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)
    np.testing.assert_allclose(dv[0, 0], np.repeat(do[0, 0].mean(axis=0, keepdims=True), N, axis=0), atol=1e-12)


def _autograd_gqa(q, k, v, do, causal, scale):
    # the grouped forward with every query head given its own copy of its KV
    # head (repeat_interleave); autograd sums the gradient over the copies
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    G = q.shape[1] // k.shape[1]
    kk, vv = t[1].repeat_interleave(G, dim=1), t[2].repeat_interleave(G, dim=1)
    s = scale * t[0] @ kk.transpose(-1, -2)
    if causal:
        n = q.shape[2]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ vv
    o.backward(torch.tensor(do))
    return [x.grad.numpy() for x in t]


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (6, 1), (8, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_matches_float64_autograd(Hq, Hkv, causal):
    B, N, d = 2, 45, 16
    q, do = (RNG.standard_normal((B, Hq, N, d)) for _ in range(2))
    k, v = (RNG.standard_normal((B, Hkv, N, d)) for _ in range(2))
    got = attention_gqa_bwd_ref(q, k, v, do, causal=causal, scale=0.3, row_block=16)
    ref = _autograd_gqa(q, k, v, do, causal, float(np.float32(0.3)))
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_one_group_is_the_square_backward(causal):
    q, k, v, do = (RNG.standard_normal((1, 3, 30, 8)) for _ in range(4))
    for g, r in zip(attention_gqa_bwd_ref(q, k, v, do, causal=causal), attention_bwd_ref(q, k, v, do, causal=causal)):
        np.testing.assert_allclose(g, r, atol=1e-13)


def test_gqa_dv_column_sum():
    # rows of P sum to 1, so summed over keys, a KV head's dV is the sum of dO
    # over all query rows of all G query heads that read it
    q, do = (RNG.standard_normal((1, 6, 20, 8)) for _ in range(2))
    k, v = (RNG.standard_normal((1, 2, 20, 8)) for _ in range(2))
    _, _, dv = attention_gqa_bwd_ref(q, k, v, do, causal=True)
    for hk in range(2):
        np.testing.assert_allclose(dv[0, hk].sum(axis=0), do[0, 3 * hk:3 * hk + 3].sum(axis=(0, 1)), atol=1e-12)
