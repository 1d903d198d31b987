"""Pins for oracle/attention.py against facts that do not come from the oracle.

Each test would fail for a plausible slip in the oracle: a transposed product
(Q K^T vs K Q^T), a dropped or squared scale, a causal off-by-one, a missing
normalisation, a wrong log base, or a dropped rescale in the online
recurrence.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention_ref, online_ref

RNG = np.random.default_rng(1234)


def _rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def _brute(q, k, v, causal, scale):
    """Scalar loops with math.fsum: softmax(scale q_i . k_j) weights on v_j."""
    B, H, N, d = q.shape
    dv = v.shape[3]
    o = np.zeros((B, H, N, dv))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                js = [j for j in range(k.shape[2]) if (not causal or j <= i)]
                s = [scale * math.fsum(q[b, h, i, t] * k[b, h, j, t] for t in range(d)) for j in js]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                z = math.fsum(w)
                for c in range(dv):
                    o[b, h, i, c] = math.fsum(w[n] * v[b, h, js[n], c] for n in range(len(js))) / z
                lse[b, h, i] = mx + math.log(z)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d,dv", [(1, 1, 1), (3, 2, 3), (5, 4, 2), (8, 4, 4)])
def test_brute_force_tiny(N, d, dv, causal):
    q, k, v = _rand(2, 2, N, d), _rand(2, 2, N, d), _rand(2, 2, N, dv)
    scale = np.float32(0.7)
    o, lse = attention_ref(q, k, v, causal=causal, scale=scale)
    ob, lb = _brute(q, k, v, causal, float(scale))
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    # with V = I the output rows are the probability rows themselves
    N = 24
    q, k = _rand(1, 2, N, 8), _rand(1, 2, N, 8)
    v = np.broadcast_to(np.eye(N), (1, 2, N, N)).copy()
    P, _ = attention_ref(q, k, v, causal=causal, scale=0.5)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-12)
    assert (P >= 0).all()
    if causal:
        assert np.all(np.triu(P[0, 0], 1) == 0) and np.all(np.triu(P[0, 1], 1) == 0)
        assert np.all(P[0, 0][np.tril_indices(N)] > 0)


def test_zero_query_gives_column_mean():
    N, d = 37, 16
    q = np.zeros((2, 3, N, d))
    k, v = _rand(2, 3, N, d), _rand(2, 3, N, d)
    o, lse = attention_ref(q, k, v, causal=False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-13)
    np.testing.assert_allclose(lse, np.full(lse.shape, math.log(N)), atol=1e-13)


def test_causal_zero_query_gives_prefix_mean():
    N, d = 29, 8
    q = np.zeros((1, 2, N, d))
    k, v = _rand(1, 2, N, d), _rand(1, 2, N, d)
    o, lse = attention_ref(q, k, v, causal=True)
    prefix = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    np.testing.assert_allclose(o, prefix, atol=1e-13)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, N + 1)), lse.shape), atol=1e-13)


def test_causal_row0_is_v0():
    N, d = 19, 8
    q, k, v = _rand(2, 2, N, d), _rand(2, 2, N, d), _rand(2, 2, N, d)
    scale = np.float32(0.3)
    o, lse = attention_ref(q, k, v, causal=True, scale=scale)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], atol=1e-14)
    np.testing.assert_allclose(lse[:, :, 0], float(scale) * (q[:, :, 0] * k[:, :, 0]).sum(-1), atol=1e-13)


def test_worked_example_closed_form():
    # N = 2, d = 1, scale = 1: S = [[0, 0], [0, 1]].
    q = np.array([0.0, 1.0]).reshape(1, 1, 2, 1)
    k = np.array([0.0, 1.0]).reshape(1, 1, 2, 1)
    v = np.eye(2).reshape(1, 1, 2, 2)
    e = math.e
    o, lse = attention_ref(q, k, v, causal=False, scale=1.0)
    np.testing.assert_allclose(o[0, 0], [[0.5, 0.5], [1 / (1 + e), e / (1 + e)]], atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], [math.log(2), math.log(1 + e)], atol=1e-15)
    o, lse = attention_ref(q, k, v, causal=True, scale=1.0)
    np.testing.assert_allclose(o[0, 0], [[1.0, 0.0], [1 / (1 + e), e / (1 + e)]], atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], [0.0, math.log(1 + e)], atol=1e-15)


def test_key_value_permutation_invariance():
    N, d = 40, 8
    q, k, v = _rand(1, 2, N, d), _rand(1, 2, N, d), _rand(1, 2, N, d)
    perm = RNG.permutation(N)
    o1, l1 = attention_ref(q, k, v)
    o2, l2 = attention_ref(q, k[:, :, perm], v[:, :, perm])
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_large_scale_tends_to_hard_max():
    N, d = 16, 4
    q, k, v = _rand(1, 1, N, d), _rand(1, 1, N, d), _rand(1, 1, N, d)
    o, _ = attention_ref(q, k, v, scale=np.float32(1e4))
    arg = np.argmax(q[0, 0] @ k[0, 0].T, axis=1)
    np.testing.assert_allclose(o[0, 0], v[0, 0, arg], atol=1e-6)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(causal):
    # a library routine: PyTorch's math path in float64 on the CPU
    B, H, N, d = 2, 3, 77, 32
    q, k, v = _rand(B, H, N, d), _rand(B, H, N, d), _rand(B, H, N, d)
    scale = np.float32(1 / math.sqrt(d))
    o, _ = attention_ref(q, k, v, causal=causal, scale=scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=float(scale))
    np.testing.assert_allclose(o, ot.numpy(), atol=1e-12)
    # logsumexp against torch.logsumexp of the explicitly masked scores
    s = float(scale) * (tq @ tk.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    _, lse = attention_ref(q, k, v, causal=causal, scale=scale)
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), atol=1e-12)


def test_rows_subset_equals_full():
    N, d = 300, 16
    q, k, v = _rand(1, 2, N, d), _rand(1, 2, N, d), _rand(1, 2, N, d)
    rows = np.array([0, 1, 63, 64, 127, 128, 255, 299])
    for causal in (False, True):
        of, lf = attention_ref(q, k, v, causal=causal, row_block=64)
        os_, ls = attention_ref(q, k, v, causal=causal, rows=rows, row_block=3)
        np.testing.assert_allclose(os_, of[:, :, rows], atol=1e-14)
        np.testing.assert_allclose(ls, lf[:, :, rows], atol=1e-14)


def test_bf16_tensor_input_is_exact():
    x = torch.randn(1, 1, 8, 4).to(torch.bfloat16)
    o1, _ = attention_ref(x, x, x)
    o2, _ = attention_ref(x.float().numpy(), x.float().numpy(), x.float().numpy())
    np.testing.assert_array_equal(o1, o2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Bc", [1, 7, 16, 64, 128, 200])
def test_online_block_size_invariance(Bc, causal):
    N, d = 200, 16
    q, k, v = _rand(2, 2, N, d) * 2, _rand(2, 2, N, d), _rand(2, 2, N, d)
    o_ref, l_ref = attention_ref(q, k, v, causal=causal, scale=0.25)
    o, l = online_ref(q, k, v, causal=causal, scale=0.25, Bc=Bc)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(l, l_ref, atol=1e-12)


def test_online_rescale_is_needed():
    # increasing scores force the running max to grow in every block; a
    # recurrence that forgot alpha would drift far from the definition
    N, d = 64, 1
    q = np.ones((1, 1, N, d))
    k = np.linspace(0, 20, N).reshape(1, 1, N, d)
    v = _rand(1, 1, N, 3)
    o_ref, _ = attention_ref(q, k, v, scale=1.0)
    o, _ = online_ref(q, k, v, scale=1.0, Bc=8)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
