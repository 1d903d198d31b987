"""GPU parity of fa_fwd_bf16_varlen (sequences of different lengths packed
end to end, token-major) against the fp64 oracle, with the gates of the bf16
forward (max-abs <= 1e-2, RMSE <= 2e-3, relative RMSE <= 1e-2, lse <= 1e-3
on rows that see keys; O = 0 and lse = -inf on rows that see none).  Lengths
include empty sequences, single rows, tile edges and sequences without keys."""

import numpy as np
import pytest
import torch

import exact_attention_73_amd as fa
from exact_attention_73_amd.inputs import make_qkv, packed_batch_lengths, softmax_scale
from oracle import attention_ref, attention_varlen_ref
from tests._util import check_rows, sample_rows

pytestmark = pytest.mark.gpu


def _packed(total_q, total_k, Hq, Hkv, d, seed):
    q, _, _ = make_qkv(1, Hq, total_q, d, seed)
    _, k, v = make_qkv(1, Hkv, total_k, d, seed + 1)
    return tuple(x[0].transpose(0, 1).contiguous() for x in (q, k, v))  # [total, H, d]


def _run(lq, lk, Hq, Hkv, d, causal, seed, max_q=None):
    cu_q, cu_k = np.cumsum([0] + lq), np.cumsum([0] + lk)
    q, k, v = _packed(int(cu_q[-1]), int(cu_k[-1]), Hq, Hkv, d, seed)
    cq = torch.tensor(cu_q, dtype=torch.int32, device="cuda")
    ck = torch.tensor(cu_k, dtype=torch.int32, device="cuda")
    mq = max(lq) if max_q is None else max_q
    o = torch.full((q.shape[0], Hq, d), float("nan"), device="cuda")
    lse = torch.full((Hq, q.shape[0]), float("nan"), device="cuda")
    fa.fwd_bf16_varlen(q.cuda(), k.cuda(), v.cuda(), cq, ck, mq, causal=causal, out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_varlen_ref(q, k, v, cu_q, cu_k, causal=causal, scale=softmax_scale(d))
    # O as [H, total, d] to line up with lse [H, total]
    check_rows(o.cpu().numpy().transpose(1, 0, 2), lse.cpu().numpy(), o_ref.transpose(1, 0, 2), lse_ref,
               f"lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    return q, k, v, cq, ck, o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_self_attention_mixed_lengths(causal):
    lens = [0, 1, 127, 128, 129, 300, 5, 1000]
    _run(lens, lens, 8, 2, 128, causal, seed=7700)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 256])
def test_varlen_head_sizes(d, causal):
    lens = [33, 0, 257, 64]
    _run(lens, lens, 4, 4, d, causal, seed=7710 + d)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_cross_lengths_and_sequences_without_keys(causal):
    # sequence 1 has three queries and no keys; sequence 2 more queries than keys
    _run([1, 3, 20, 17], [100, 0, 5, 400], 6, 1, 128, causal, seed=7720)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_pingpong_lengths(causal):
    # longest sequence >= 1024 rows at d = 128: 256-row workgroups of eight
    # waves; lengths straddle their edges, keys longer and shorter than queries
    lq = [1100, 0, 1, 255, 257, 2049, 700]
    lk = [1100, 0, 1, 255, 300, 2049, 650]
    _run(lq, lk, 4, 2, 128, causal, seed=7750)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_pingpong_sequences_without_keys(causal):
    # rows past every key of their sequence, a sequence with no keys at all
    _run([1030, 3, 600, 513], [70, 0, 1500, 513], 3, 1, 128, causal, seed=7760)


def test_varlen_grid_larger_than_needed():
    _run([50, 70], [50, 70], 2, 1, 128, True, seed=7730, max_q=1000)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [300, 1100])
def test_varlen_equal_lengths_match_fixed_length_forward(N, causal):
    # three sequences of N: the same per-tile work as the [B, H, N, d] call, bit
    # for bit (N = 1100: both take the 256-row ping-pong workgroups)
    B, Hq, Hkv, d = 3, 4, 2, 128
    q, _, _ = make_qkv(B, Hq, N, d, 7740 + N)
    _, k, v = make_qkv(B, Hkv, N, d, 7741 + N)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o4, l4 = fa.fwd_bf16_gqa(qd, kd, vd, causal=causal)
    pack = lambda x: x.transpose(1, 2).reshape(B * N, x.shape[1], d).contiguous()
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
    o, lse = fa.fwd_bf16_varlen(pack(qd), pack(kd), pack(vd), cu, cu, N, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o4.transpose(1, 2).reshape(B * N, Hq, d))
    assert torch.equal(lse, l4.permute(1, 0, 2).reshape(Hq, B * N))


def test_varlen_packed_workload_sampled():
    """The packed batch bench.py times (16 causal sequences of 256..4096
    tokens, 36194 in all, H16 d128, the ping-pong kernel), in the same launch:
    sampled rows of every sequence, on three heads, against the oracle run
    on each sequence alone."""
    lens = packed_batch_lengths()
    H, d = 16, 128
    tot = sum(lens)
    q, _, _ = make_qkv(1, H, tot, d, 73801)
    _, k, v = make_qkv(1, H, tot, d, 73802)
    q, k, v = (x[0].transpose(0, 1).contiguous() for x in (q, k, v))  # [total, H, d]
    cu = np.cumsum([0] + lens)
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    o, lse = fa.fwd_bf16_varlen(q.cuda(), k.cuda(), v.cuda(), cu_d, cu_d, max(lens), causal=True)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    sc = softmax_scale(d)
    for s_, n in enumerate(lens):
        a = int(cu[s_])
        rows = sample_rows(n, extra=8, seed=s_)
        for h in (0, 7, H - 1):
            seq = lambda x: x[a:a + n, h][None, None]  # [1, 1, n, d]
            o_ref, lse_ref = attention_ref(seq(q), seq(k), seq(v), causal=True, scale=sc, rows=rows)
            check_rows(o[a + rows, h][None, None], lse[h, a + rows][None, None], o_ref, lse_ref,
                       f"packed workload seq {s_} (n={n}) head {h}")
