"""GPU parity of fa_fwd_bf16_decode (packed query heads, split-KV, chunk
merge) against the fp64 oracle of grouped-query attention, with the gates
of the bf16 forward (max-abs <= 1e-2, RMSE <= 2e-3, relative RMSE <= 1e-2,
lse <= 1e-3 on rows that see keys; O = 0 and lse = -inf on rows that see
none).  The split count is forced over 1, a few, one per tile and the cost
model's choice, so every path of the merge is compared."""

import pytest
import torch

import exact_attention_73_amd as fa
from exact_attention_73_amd.inputs import make_qkv, softmax_scale
from oracle import attention_gqa_ref
from tests._util import check_rows

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, Nq, Nk, d, seed):
    q, _, _ = make_qkv(B, Hq, Nq, d, seed)
    _, k, v = make_qkv(B, Hkv, Nk, d, seed + 1)
    return q, k, v


def _check(B, Hq, Hkv, Nq, Nk, d, causal, splits, seed):
    q, k, v = _inputs(B, Hq, Hkv, Nq, Nk, d, seed)
    o, lse = fa.fwd_bf16_decode(q.cuda(), k.cuda(), v.cuda(), causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_gqa_ref(q, k, v, causal=causal, scale=softmax_scale(d))
    used = fa.decode_splits(B, Hq, Hkv, Nq, Nk, d, splits)
    check_rows(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref,
               f"B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} splits={splits}->{used}")


SHAPES = [
    # B, Hq, Hkv, Nq, Nk, d
    (2, 4, 4, 1, 1000, 128),   # multi-head decode, one query
    (1, 8, 2, 1, 3001, 128),   # grouped heads, ragged tail tile
    (2, 32, 8, 4, 2049, 128),  # 4 heads x 4 queries = 16 packed rows
    (1, 16, 1, 5, 1500, 128),  # multi-query: 80 packed rows, three row blocks
    (1, 16, 1, 3, 777, 64),
    (1, 4, 2, 2, 999, 256),
    (1, 2, 1, 1, 5, 64),       # fewer keys than one tile
    (1, 4, 2, 70, 50, 128),    # more queries than keys: causal rows with no key
]


@pytest.mark.parametrize("splits", [0, 1, 3, 1000])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}".format(*s))
def test_decode_shapes(shape, causal, splits):
    B, Hq, Hkv, Nq, Nk, d = shape
    _check(B, Hq, Hkv, Nq, Nk, d, causal, splits, seed=7300 + Nq + Nk + d)


@pytest.mark.parametrize("Nk", [8192, 32768])
def test_decode_serving_shape(Nk):
    # 32 query heads over 8 KV heads, one new token per sequence, the cost
    # model's split count (several chunks at these sizes)
    _check(4, 32, 8, 1, Nk, 128, True, 0, seed=7400)


def test_decode_matches_across_split_counts():
    # different chunkings of the same keys agree closely with each other
    q, k, v = (x.cuda() for x in _inputs(1, 8, 1, 2, 4000, 128, seed=7500))
    o1, l1 = fa.fwd_bf16_decode(q, k, v, num_splits=1)
    for s in (2, 5, 17, 125):
        o, l = fa.fwd_bf16_decode(q, k, v, num_splits=s)
        assert float((o - o1).abs().max()) <= 2e-3 and float((l - l1).abs().max()) <= 1e-4, s


def test_decode_workspace_checks():
    q, k, v = (x.cuda() for x in _inputs(1, 4, 1, 1, 4096, 128, seed=7600))
    splits = fa.decode_splits(1, 4, 1, 1, 4096, 128, 8)
    assert splits == 8
    need = fa.decode_workspace_bytes(1, 4, 1, 128, splits)
    assert need == 8 * 4 * 129 * 4
    small = torch.empty(need // 4 - 1, dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FaError) as ei:
        fa.fwd_bf16_decode(q, k, v, num_splits=8, workspace=small)
    assert ei.value.status == -8
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")  # contents do not matter
    o, lse = fa.fwd_bf16_decode(q, k, v, num_splits=8, workspace=ws)
    o_ref, lse_ref = attention_gqa_ref(*(x.cpu() for x in (q, k, v)), scale=softmax_scale(128))
    torch.cuda.synchronize()
    check_rows(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "preset workspace")
