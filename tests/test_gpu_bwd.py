"""GPU parity of fa_bwd_bf16 (dQ, dK, dV) against the fp64 oracle.

The GPU backward recomputes P from bf16 Q, K with the forward's fp32 lse and
rounds P and dS to bf16 for its matrix products (relative 2^-9 per
element); dV, dK, dQ are sums of such terms with fp32 accumulation.  Gates,
per gradient against the fp64 gradients of the same bf16 inputs: relative
RMSE <= 1e-2 and max-abs error <= 2e-2 of the largest reference magnitude.
"""

import numpy as np
import pytest
import torch

import exact_attention_73_amd as fa
from exact_attention_73_amd.inputs import WORKLOADS, make_do, make_qkv, softmax_scale
from oracle import attention_bwd_ref
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
        big = float(np.abs(r).max()) or 1.0
        print(f"{label} {name}: {e}")
        assert e["rel_rmse"] <= 1e-2, (label, name, e)
        assert e["max_abs"] <= 2e-2 * big, (label, name, e)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 127, 128, 129, 200, 255, 300])
def test_bwd_edges(N, d, causal):
    q, k, v = make_qkv(1, 2, N, d, seed=6000 + N + d)
    do = make_do(1, 2, N, d, seed=6000 + N + d)
    got = _run(q, k, v, do, causal)
    ref = attention_bwd_ref(q, k, v, do, causal=causal, scale=softmax_scale(d))
    _check(got, ref, f"N={N} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_multi_tile(causal):
    q, k, v = make_qkv(2, 4, 1000, 128, seed=6100)
    do = make_do(2, 4, 1000, 128, seed=6100)
    got = _run(q, k, v, do, causal)
    ref = attention_bwd_ref(q, k, v, do, causal=causal, scale=softmax_scale(128))
    _check(got, ref, f"B2 H4 N1000 causal={causal}")


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


def test_bwd_deterministic():
    q, k, v = make_qkv(1, 4, 777, 128, seed=6200)
    do = make_do(1, 4, 777, 128, seed=6200)
    a = _run(q, k, v, do, True)
    b = _run(q, k, v, do, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_invalid_arguments():
    q, k, v = (x.cuda() for x in make_qkv(1, 1, 64, 256, seed=1))
    o = torch.zeros(1, 1, 64, 256, device="cuda")
    lse = torch.zeros(1, 1, 64, device="cuda")
    with pytest.raises(fa.FaError) as ei:
        fa.bwd_bf16(q, k, v, o, lse, q)
    assert ei.value.status == -3
