"""Asynchronous-boundary checks of the forward (FA3 explainer, section
"正确性验证要覆盖异步边界": races between barriers and buffer reuse, and
graph capture, are among what tests must cover).

* Stress: 1000 back-to-back launches of the d = 128 ping-pong forward on the
  standard block (B4 H16 N2048 d128), alternating non-causal and causal,
  each compared bitwise with the first launch of its kind (checked every 50
  launches, stopping at the first mismatch).  The ping-pong kernel's phase
  switch is a barrier without a memory fence, so a timing-dependent race in
  the ring would show as a run-to-run difference.
* Graph capture: the forward captured in a torch CUDA graph (HIP graph) and
  replayed several times, with eager work that changes the inputs between
  replays; every replay must equal an eager launch on the same inputs.
* Binding: caller-supplied outputs of the wrong shape are rejected before
  any launch.
"""

import pytest
import torch

import exact_attention_73_amd as fa
from exact_attention_73_amd.inputs import WORKLOADS, make_qkv

pytestmark = pytest.mark.gpu


def test_pingpong_stress_bitwise(gpu_lib):
    w = WORKLOADS["std"]
    q, k, v = (x.cuda() for x in make_qkv(w.B, w.H, w.N, w.d, w.seed))
    ref = {c: fa.fwd_bf16(q, k, v, causal=c) for c in (False, True)}
    outs = {c: (torch.empty_like(ref[c][0]), torch.empty_like(ref[c][1])) for c in (False, True)}
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    done = 0
    for chunk in range(20):
        for i in range(50):
            c = bool(i & 1)
            o, l = outs[c]
            fa.fwd_bf16(q, k, v, causal=c, out=o, lse=l)
            bad += (o != ref[c][0]).sum() + (l != ref[c][1]).sum()
        done += 50
        torch.cuda.synchronize()
        assert int(bad) == 0, f"mismatch within launches {done - 50}..{done - 1}"
    print(f"{done} launches bitwise equal")


@pytest.mark.parametrize("N,d", [(2048, 128), (1000, 128), (600, 64), (300, 256)])
@pytest.mark.parametrize("causal", [False, True])
def test_graph_capture_replay(gpu_lib, N, d, causal):
    B, H = 2, 4
    srcs = [tuple(x.cuda() for x in make_qkv(B, H, N, d, seed=8800 + i)) for i in range(3)]
    q, k, v = (x.clone() for x in srcs[0])
    o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    eager = [fa.fwd_bf16(*s, causal=causal) for s in srcs]
    fa.fwd_bf16(q, k, v, causal=causal, out=o, lse=lse)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            fa.fwd_bf16(q, k, v, causal=causal, out=o, lse=lse)
    torch.cuda.synchronize()
    for rep in range(6):
        i = rep % 3
        for dst, src in zip((q, k, v), srcs[i]):
            dst.copy_(src)  # eager work between replays
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager[i][0]) and torch.equal(lse, eager[i][1]), f"replay {rep}"


def test_undersized_outputs_rejected(gpu_lib):
    q, k, v = (x.cuda() for x in make_qkv(1, 2, 100, 128, seed=8900))
    with pytest.raises(ValueError):
        fa.fwd_bf16(q, k, v, out=torch.empty((1, 2, 99, 128), device="cuda"))
    with pytest.raises(ValueError):
        fa.fwd_bf16(q, k, v, lse=torch.empty((1, 2, 99), device="cuda"))
    with pytest.raises(ValueError):
        fa.fwd_bf16_gqa(q, k[:, :1].contiguous(), v[:, :1].contiguous(), out=torch.empty((2, 100, 128), device="cuda"))
    with pytest.raises(ValueError):
        fa.fwd_bf16_decode(q[:, :, :1].contiguous(), k, v, lse=torch.empty((1, 2), device="cuda"))
    qt, kt, vt = (x[0].transpose(0, 1).contiguous() for x in (q, k, v))
    cu = torch.tensor([0, 40, 100], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        fa.fwd_bf16_varlen(qt, kt, vt, cu, cu, 60, lse=torch.empty((2, 99), device="cuda"))
    signs = torch.ones((2, 128), dtype=torch.int8, device="cuda")
    q8, qs = fa.fp8_prep(q, signs=signs)
    k8, ks = fa.fp8_prep(k, signs=signs)
    v8t, vs = fa.fp8_prep_v(v)
    with pytest.raises(ValueError):
        fa.fwd_fp8(q8, k8, v8t, qs, ks, vs, out=torch.empty((1, 2, 100, 127), device="cuda"))
    with pytest.raises(ValueError):
        fa.fp8_prep(q, signs=signs, out=torch.empty((1, 2, 100, 127), dtype=torch.uint8, device="cuda"))
