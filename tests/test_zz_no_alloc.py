"""fa_fwd_bf16_decode_noalloc, the decode forward that allocates nothing
(its chunk partials live in the library's static per-device scratch
buffer), against fa_fwd_bf16_decode with a caller workspace: the same
kernels with the same effective split count, so the outputs must be
bit-identical.  Two calls in a row, the second with a smaller input (the
buffer keeps the first call's partials), the library's own split choice,
and the rejection of a split count whose partials do not fit."""

import pytest
import torch

import exact_attention_73_amd as fa
from exact_attention_73_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, Nq, Nk, d, seed):
    q, _, _ = make_qkv(B, Hq, Nq, d, seed)
    _, k, v = make_qkv(B, Hkv, Nk, d, seed + 1)
    return q.cuda(), k.cuda(), v.cuda()


def _compare(shape, causal, splits, seed):
    B, Hq, Hkv, Nq, Nk, d = shape
    q, k, v = _inputs(B, Hq, Hkv, Nq, Nk, d, seed)
    o_ref, l_ref = fa.fwd_bf16_decode(q, k, v, causal=causal, num_splits=splits)
    o = torch.full((B, Hq, Nq, d), float("nan"), device="cuda")
    lse = torch.full((B, Hq, Nq), float("nan"), device="cuda")
    fa.fwd_bf16_decode_noalloc(q, k, v, causal=causal, num_splits=splits, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), (shape, causal, splits)


def test_noalloc_two_calls_second_smaller(gpu_lib):
    # 1024 packed rows x 8 chunks x 129 floats = 4.2 MB of partials, then a
    # smaller call that reuses the front of the same buffer
    _compare((8, 32, 8, 4, 8192, 128), True, 8, 9500)
    _compare((2, 8, 2, 2, 3000, 128), False, 3, 9510)


def test_noalloc_library_split_choice_and_head_sizes(gpu_lib):
    for shape, causal in (((4, 32, 8, 1, 32768, 128), True), ((1, 16, 1, 3, 777, 64), False),
                          ((1, 4, 2, 2, 999, 256), True)):
        B, Hq, Hkv, Nq, Nk, d = shape
        used = fa.decode_splits(B, Hq, Hkv, Nq, Nk, d)
        assert used * B * Hq * Nq * (d + 1) * 4 <= 16 << 20
        _compare(shape, causal, used, 9520 + d)  # the workspace entry point at the count the model picks
        q, k, v = _inputs(B, Hq, Hkv, Nq, Nk, d, 9520 + d)
        a = fa.fwd_bf16_decode(q, k, v, causal=causal, num_splits=0)
        b = fa.fwd_bf16_decode_noalloc(q, k, v, causal=causal, num_splits=0)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_noalloc_rejects_partials_beyond_the_buffer(gpu_lib):
    q, k, v = _inputs(8, 32, 8, 4, 8192, 128, 9530)
    o = torch.full((8, 32, 4, 128), 7.0, device="cuda")
    lse = torch.full((8, 32, 4), 7.0, device="cuda")
    # 64 chunks x 1024 rows x 129 floats = 33.8 MB > 16 MiB
    with pytest.raises(fa.FaError) as ei:
        fa.fwd_bf16_decode_noalloc(q, k, v, num_splits=64, out=o, lse=lse)
    assert ei.value.status == -9
    torch.cuda.synchronize()
    assert (o == 7.0).all() and (lse == 7.0).all()
    # the library's own choice for the same shape fits and matches
    a = fa.fwd_bf16_decode(q, k, v, num_splits=0)
    fa.fwd_bf16_decode_noalloc(q, k, v, num_splits=0, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    ref = fa.fwd_bf16_gqa(q, k, v)
    torch.cuda.synchronize()
    assert float((o - ref[0]).abs().max()) <= 1e-2
