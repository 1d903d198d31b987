"""GPU parity of fa_bwd_bf16 (dQ, dK, dV) against the fp64 oracle.

The GPU backward recomputes P from bf16 Q, K with the forward's fp32 lse and
rounds P and dS to bf16 for its matrix products (relative 2^-8 per
element); dV, dK, dQ are sums of such terms with fp32 accumulation.  Gates,
per gradient against the fp64 gradients of the same bf16 inputs: relative
RMSE <= 1e-2 and max-abs error <= 2e-2 of the largest reference magnitude.
"""

import numpy as np
import pytest
import torch

import exact_attention_73_amd as fa
from exact_attention_73_amd.inputs import WORKLOADS, make_do, make_qkv, softmax_scale
from oracle import attention_bwd_ref, attention_gqa_bwd_ref
from tests._util import errors

pytestmark = pytest.mark.gpu


def _run(q, k, v, do, causal):
    qc, kc, vc, dc = (x.cuda() for x in (q, k, v, do))
    o, lse = fa.fwd_bf16(qc, kc, vc, causal=causal)
    dq, dk, dv = fa.bwd_bf16(qc, kc, vc, o, lse, dc, causal=causal)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


def _check(got, ref, label):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.isfinite(g).all(), (label, name)
        e = errors(g, r)
        big = float(np.abs(r).max())
        print(f"{label} {name}: {e}")
        if big == 0.0:
            # an exactly zero gradient (one visible key: softmax 1, so dS = P (dP - D) = 0):
            # the GPU forms dP with the matrix cores and D = rowsum(dO * O) in another
            # fp32 order, so dS keeps residues of fp32 rounding (2^-24 of |dP|)
            assert e["max_abs"] <= 1e-5, (label, name, e)
            continue
        assert e["rel_rmse"] <= 1e-2, (label, name, e)
        assert e["max_abs"] <= 2e-2 * big, (label, name, e)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 127, 128, 129, 200, 255, 300])
def test_bwd_edges(N, d, causal):
    q, k, v = make_qkv(1, 2, N, d, seed=6000 + N + d)
    do = make_do(1, 2, N, d, seed=6000 + N + d)
    got = _run(q, k, v, do, causal)
    ref = attention_bwd_ref(q, k, v, do, causal=causal, scale=softmax_scale(d))
    _check(got, ref, f"N={N} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [128, 256])
def test_bwd_multi_tile(causal, d):
    q, k, v = make_qkv(2, 4, 1000, d, seed=6100)
    do = make_do(2, 4, 1000, d, seed=6100)
    got = _run(q, k, v, do, causal)
    ref = attention_bwd_ref(q, k, v, do, causal=causal, scale=softmax_scale(d))
    _check(got, ref, f"B2 H4 N1000 d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_std_block_sampled_heads(causal):
    w = WORKLOADS["std"]
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.seed)
    do = make_do(w.B, w.H, w.N, w.d, w.seed)
    dq, dk, dv = _run(q, k, v, do, causal)
    for b, h in ((0, 0), (3, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = attention_bwd_ref(q[sl], k[sl], v[sl], do[sl], causal=causal, scale=softmax_scale(w.d))
        _check((dq[sl], dk[sl], dv[sl]), ref, f"std b={b} h={h} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_split_launches_match_single_launch(causal):
    # B4 H16 N1000 d128 fills the device (512 workgroups of 128 keys), so dK
    # and dV come from two launches; head 0 alone (8 workgroups) takes the
    # single dK/dV launch.  Same arithmetic in the same order: equal bit for bit.
    q, k, v = (x.cuda() for x in make_qkv(4, 16, 1000, 128, seed=6300))
    do = make_do(4, 16, 1000, 128, seed=6300).cuda()
    o, lse = fa.fwd_bf16(q, k, v, causal=causal)
    big = fa.bwd_bf16(q, k, v, o, lse, do, causal=causal)
    one = [x[:1, :1].contiguous() for x in (q, k, v, o, lse, do)]
    small = fa.bwd_bf16(*one, causal=causal)
    torch.cuda.synchronize()
    for g_big, g_small in zip(big, small):
        assert torch.equal(g_big[:1, :1], g_small)
    # and the tiled tail against the oracle on a sampled head
    ref = attention_bwd_ref(q[1:2, 5:6].cpu(), k[1:2, 5:6].cpu(), v[1:2, 5:6].cpu(), do[1:2, 5:6].cpu(), causal=causal,
                            scale=softmax_scale(128))
    _check(tuple(g[1:2, 5:6].cpu().numpy() for g in big), ref, f"split launches causal={causal}")


def _gqa_inputs(B, Hq, Hkv, N, d, seed):
    q, _, _ = make_qkv(B, Hq, N, d, seed)
    _, k, v = make_qkv(B, Hkv, N, d, seed + 1)
    return q, k, v, make_do(B, Hq, N, d, seed)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(1, 4, 2, 300, 128), (1, 6, 1, 129, 64), (2, 8, 2, 1000, 128),
                                           (1, 4, 4, 200, 64), (1, 8, 1, 64, 128), (1, 4, 2, 300, 256)])
def test_bwd_gqa_against_oracle(B, Hq, Hkv, N, d, causal):
    q, k, v, do = _gqa_inputs(B, Hq, Hkv, N, d, seed=6400 + N + d + Hq)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.fwd_bf16_gqa(qd, kd, vd, causal=causal)
    got = fa.bwd_bf16_gqa(qd, kd, vd, o, lse, dod, causal=causal)
    torch.cuda.synchronize()
    ref = attention_gqa_bwd_ref(q, k, v, do, causal=causal, scale=softmax_scale(d))
    _check(tuple(g.cpu().numpy() for g in got), ref, f"gqa B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_gqa_split_launches_sampled(causal):
    # 4 x 8 KV heads x 8 key tiles = 256 workgroups: dK/dV take the two-launch path
    B, Hq, Hkv, N, d = 4, 32, 8, 1000, 128
    q, k, v, do = _gqa_inputs(B, Hq, Hkv, N, d, seed=6500)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.fwd_bf16_gqa(qd, kd, vd, causal=causal)
    dq, dk, dv = fa.bwd_bf16_gqa(qd, kd, vd, o, lse, dod, causal=causal)
    torch.cuda.synchronize()
    for b, hk in ((0, 0), (3, 5)):
        hs = slice(4 * hk, 4 * hk + 4)
        ref = attention_gqa_bwd_ref(q[b:b + 1, hs], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1], do[b:b + 1, hs],
                                    causal=causal, scale=softmax_scale(d))
        got = (dq[b:b + 1, hs].cpu().numpy(), dk[b:b + 1, hk:hk + 1].cpu().numpy(), dv[b:b + 1, hk:hk + 1].cpu().numpy())
        _check(got, ref, f"gqa split b={b} kv head={hk} causal={causal}")


def test_bwd_gqa_consistent_with_expanded_heads():
    # dQ equals the ungrouped backward on K, V copied to every query head (the
    # same kernel work per query head: bit for bit); dK, dV equal the sums of
    # the copies' gradients up to the order of the fp32 sums
    B, Hq, Hkv, N, d = 1, 6, 2, 257, 128
    q, k, v, do = (x.cuda() for x in _gqa_inputs(B, Hq, Hkv, N, d, seed=6600))
    o, lse = fa.fwd_bf16_gqa(q, k, v, causal=True)
    dq, dk, dv = fa.bwd_bf16_gqa(q, k, v, o, lse, do, causal=True)
    ke, ve = (x.repeat_interleave(Hq // Hkv, dim=1).contiguous() for x in (k, v))
    dq1, dk1, dv1 = fa.bwd_bf16(q, ke, ve, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq1)
    for g, g1 in ((dk, dk1), (dv, dv1)):
        s = g1.reshape(B, Hkv, Hq // Hkv, N, d).sum(2)
        assert float((g - s).abs().max()) <= 1e-4 * float(s.abs().max())
    # one group per KV head is the ungrouped backward exactly
    q2, k2, v2 = q[:, :2].contiguous(), k, v
    o2, l2 = fa.fwd_bf16(q2, k2, v2, causal=True)
    a = fa.bwd_bf16_gqa(q2, k2, v2, o2, l2, do[:, :2].contiguous(), causal=True)
    b_ = fa.bwd_bf16(q2, k2, v2, o2, l2, do[:, :2].contiguous(), causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b_))


def test_bwd_deterministic():
    q, k, v = make_qkv(1, 4, 777, 128, seed=6200)
    do = make_do(1, 4, 777, 128, seed=6200)
    a = _run(q, k, v, do, True)
    b = _run(q, k, v, do, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_invalid_arguments():
    q, k, v = (x.cuda() for x in make_qkv(1, 1, 64, 96, seed=1))
    o = torch.zeros(1, 1, 64, 96, device="cuda")
    lse = torch.zeros(1, 1, 64, device="cuda")
    with pytest.raises(fa.FaError) as ei:
        fa.bwd_bf16(q, k, v, o, lse, q)
    assert ei.value.status == -3
