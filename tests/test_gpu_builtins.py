"""In-bounds checks of the gfx950 builtins whose lane layout or rounding the
kernels depend on (one wave each, a few KB of buffers)."""

import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_encode

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(__file__), "hip", "libprobes.so")


@pytest.fixture(scope="module")
def probes():
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    lib = ctypes.CDLL(LIB)
    for n in ("probe_mfma_bf16", "probe_mfma_fp8", "probe_mfma_fp8_lanescale", "probe_mfma_fp8_unscaled",
              "probe_cvt_fp8", "probe_swap_halves", "probe_tr16", "probe_load_lds"):
        getattr(lib, n).restype = ctypes.c_int
    return lib


def _s():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_mfma_bf16_32x32x16_layout(probes):
    g = torch.Generator().manual_seed(1)
    A = torch.randn(32, 16, generator=g).to(torch.bfloat16)
    B = torch.randn(16, 32, generator=g).to(torch.bfloat16)
    a = torch.empty(64, 8, dtype=torch.bfloat16)
    b = torch.empty(64, 8, dtype=torch.bfloat16)
    for l in range(64):
        a[l] = A[l % 32, 8 * (l // 32): 8 * (l // 32) + 8]
        b[l] = B[8 * (l // 32): 8 * (l // 32) + 8, l % 32]
    c = torch.zeros(64, 16, dtype=torch.float32, device="cuda")
    assert probes.probe_mfma_bf16(_p(a.cuda()), _p(b.cuda()), _p(c), _s()) == 0
    torch.cuda.synchronize()
    c = c.cpu().numpy()
    ref = A.double().numpy() @ B.double().numpy()
    got = np.zeros((32, 32))
    for l in range(64):
        for r in range(16):
            got[8 * (r // 4) + 4 * (l // 32) + (r % 4), l % 32] = c[l, r]
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("sa,sb", [(127, 127), (120, 130), (133, 120)])
def test_mfma_fp8_32x32x64_layout_and_scales(probes, sa, sb):
    rng = np.random.default_rng(sa * 1000 + sb)
    A = rng.integers(0, 256, size=(32, 64)).astype(np.uint8)
    B = rng.integers(0, 256, size=(64, 32)).astype(np.uint8)
    A[(A & 0x7F) == 0x7F] = 0x38  # no NaN codes
    B[(B & 0x7F) == 0x7F] = 0x38
    a = np.zeros((64, 32), np.uint8)
    b = np.zeros((64, 32), np.uint8)
    for l in range(64):
        a[l] = A[l % 32, 32 * (l // 32): 32 * (l // 32) + 32]
        b[l] = B[32 * (l // 32): 32 * (l // 32) + 32, l % 32]
    c = torch.zeros(64, 16, dtype=torch.float32, device="cuda")
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    assert probes.probe_mfma_fp8(_p(ta), _p(tb), _p(c), sa, sb, _s()) == 0
    torch.cuda.synchronize()
    c = c.cpu().numpy()
    ref = (e4m3_decode(A) @ e4m3_decode(B)) * 2.0 ** (sa - 127) * 2.0 ** (sb - 127)
    got = np.zeros((32, 32))
    for l in range(64):
        for r in range(16):
            got[8 * (r // 4) + 4 * (l // 32) + (r % 4), l % 32] = c[l, r]
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-3 * np.abs(ref).max())


def test_mfma_fp8_per_lane_scales(probes):
    """Per-lane E8M0 scales: with lane L holding bytes j = 0..31 of row/column
    L % 32 (k = 32 (L // 32) + j, the layout the products above verify), byte
    j takes the scale of lane (L % 32) + 32 (j // 16) -- bytes 0..15 the
    first half-wave's, bytes 16..31 the second's.  So equal scales in lanes
    n and n + 32 scale column n (or row n) of the product exactly, which is
    what the FP8 forward relies on for its per-query-row power of two."""
    rng = np.random.default_rng(11)
    A = rng.integers(0, 256, size=(32, 64)).astype(np.uint8)
    B = rng.integers(0, 256, size=(64, 32)).astype(np.uint8)
    A[(A & 0x7F) == 0x7F] = 0x38
    B[(B & 0x7F) == 0x7F] = 0x38
    sa = rng.integers(120, 135, size=64).astype(np.int32)
    sb = rng.integers(110, 140, size=64).astype(np.int32)
    a = np.zeros((64, 32), np.uint8)
    b = np.zeros((64, 32), np.uint8)
    for l in range(64):
        a[l] = A[l % 32, 32 * (l // 32): 32 * (l // 32) + 32]
        b[l] = B[32 * (l // 32): 32 * (l // 32) + 32, l % 32]
    c = torch.zeros(64, 16, dtype=torch.float32, device="cuda")
    assert probes.probe_mfma_fp8_lanescale(_p(torch.from_numpy(a).cuda()), _p(torch.from_numpy(b).cuda()), _p(c),
                                           _p(torch.from_numpy(sa).cuda()), _p(torch.from_numpy(sb).cuda()), _s()) == 0
    torch.cuda.synchronize()
    cc = c.cpu().numpy()
    got = np.zeros((32, 32))
    for l in range(64):
        for r in range(16):
            got[8 * (r // 4) + 4 * (l // 32) + (r % 4), l % 32] = cc[l, r]
    sel = (np.arange(64) % 32) // 16  # which half-wave's scale byte k takes
    Ad = e4m3_decode(A) * 2.0 ** (sa[np.arange(32)[:, None] + 32 * sel[None, :]] - 127)
    Bd = e4m3_decode(B) * 2.0 ** (sb[np.arange(32)[None, :] + 32 * sel[:, None]] - 127)
    ref = Ad @ Bd
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-4 * np.abs(ref).max())
    # the property the forward kernel uses: equal scales in both halves
    sb2 = np.concatenate([sb[:32], sb[:32]]).astype(np.int32)
    c2 = torch.zeros(64, 16, dtype=torch.float32, device="cuda")
    assert probes.probe_mfma_fp8_lanescale(_p(torch.from_numpy(a).cuda()), _p(torch.from_numpy(b).cuda()), _p(c2),
                                           _p(torch.from_numpy(np.full(64, 127, np.int32)).cuda()),
                                           _p(torch.from_numpy(sb2).cuda()), _s()) == 0
    torch.cuda.synchronize()
    cc = c2.cpu().numpy()
    for l in range(64):
        for r in range(16):
            got[8 * (r // 4) + 4 * (l // 32) + (r % 4), l % 32] = cc[l, r]
    ref2 = (e4m3_decode(A) @ e4m3_decode(B)) * 2.0 ** (sb[None, :32] - 127)
    np.testing.assert_allclose(got, ref2, rtol=1e-5, atol=1e-4 * np.abs(ref2).max())


def test_mfma_fp8_unscaled_form(probes):
    # scale operands 0 select the plain instruction; record what it computes
    rng = np.random.default_rng(7)
    A = (rng.integers(0, 2, size=(32, 64)) * 0x38).astype(np.uint8)  # 0 or 1.0
    B = (rng.integers(0, 2, size=(64, 32)) * 0x38).astype(np.uint8)
    a = np.zeros((64, 32), np.uint8)
    b = np.zeros((64, 32), np.uint8)
    for l in range(64):
        a[l] = A[l % 32, 32 * (l // 32): 32 * (l // 32) + 32]
        b[l] = B[32 * (l // 32): 32 * (l // 32) + 32, l % 32]
    c = torch.zeros(64, 16, dtype=torch.float32, device="cuda")
    assert probes.probe_mfma_fp8_unscaled(_p(torch.from_numpy(a).cuda()), _p(torch.from_numpy(b).cuda()), _p(c), _s()) == 0
    torch.cuda.synchronize()
    ref = e4m3_decode(A) @ e4m3_decode(B)
    got = np.zeros((32, 32))
    cc = c.cpu().numpy()
    for l in range(64):
        for r in range(16):
            got[8 * (r // 4) + 4 * (l // 32) + (r % 4), l % 32] = cc[l, r]
    print("unscaled fp8 mfma / exact product ratio:", float(got.sum() / max(ref.sum(), 1)))
    np.testing.assert_allclose(got, ref, rtol=1e-6)


def test_cvt_pk_fp8_rounding_matches_oracle(probes):
    vals = e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (vals[1:] + vals[:-1]) / 2
    rng = np.random.default_rng(3)
    x = np.concatenate([vals, -vals, mids, -mids, rng.uniform(-448, 448, 4000), rng.normal(0, 0.01, 4000)])
    x = x[: (len(x) // 4) * 4].astype(np.float32)
    n = len(x) // 4
    out = torch.zeros(n, dtype=torch.int32, device="cuda")
    assert probes.probe_cvt_fp8(_p(torch.from_numpy(x).cuda()), _p(out), n, _s()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint8).reshape(-1)
    np.testing.assert_array_equal(e4m3_decode(got), e4m3_decode(e4m3_encode(x.astype(np.float64))))


def test_swap_halves(probes):
    # v_permlane32_swap: lanes 32..63 of the first operand trade places with
    # lanes 0..31 of the second; max and sum of the two results combine each
    # lane's value with the other half-wave's, bit-identically in both halves
    xh = (np.arange(64, dtype=np.float32) * 1.37 - 40.0).astype(np.float32)
    xh[[3, 40]] = [1e-3, -7.25]
    x = torch.from_numpy(xh).cuda()
    y = torch.zeros(4 * 64, dtype=torch.float32, device="cuda")
    assert probes.probe_swap_halves(_p(x), _p(y), _s()) == 0
    torch.cuda.synchronize()
    a, b, mx, sm = y.cpu().numpy().reshape(4, 64)
    lane = np.arange(64)
    np.testing.assert_array_equal(a, np.where(lane < 32, xh, xh[lane ^ 32]))
    np.testing.assert_array_equal(b, np.where(lane < 32, xh[lane ^ 32], xh))
    np.testing.assert_array_equal(mx, np.maximum(xh, xh[lane ^ 32]))
    np.testing.assert_array_equal(sm, (xh + xh[lane ^ 32]).astype(np.float32))


def test_ds_read_tr16_b64_mapping(probes):
    # informational: record which LDS element each lane receives when lane l
    # addresses the 64-bit row at byte 8 l
    addr = torch.arange(64, dtype=torch.int32, device="cuda") * 8
    out = torch.zeros(64 * 4, dtype=torch.int16, device="cuda")
    assert probes.probe_tr16(_p(addr), _p(out), _s()) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy().reshape(64, 4)
    os.makedirs("gpurun_out", exist_ok=True)
    with open("gpurun_out/tr16_mapping.txt", "w") as f:
        for l in range(64):
            f.write(f"{l}: {list(map(int, o[l]))}\n")
    print("tr16 lane 0..3:", o[:4].tolist())
    assert o.min() >= 0 and o.max() < 256


def test_buffer_load_lds_placement_and_range(probes):
    # lane l loads 16 bytes from a permuted offset; they land at LDS base
    # + 16 l; offsets at or past the buffer's range read as zero
    src = torch.arange(512, dtype=torch.int32, device="cuda")  # 2 KB of distinct words
    perm = np.random.default_rng(0).permutation(64)
    off = (perm * 16).astype(np.int32)
    off[60:] = [1024, 1040, 2048, 4096]  # beyond nbytes = 1024: zero
    out = torch.zeros(320, dtype=torch.int32, device="cuda")
    assert probes.probe_load_lds(_p(src), _p(torch.from_numpy(off).cuda()), 1024, _p(out), _s()) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint32)
    assert np.all(o[:16] == 0xDEADBEEF) and np.all(o[16 + 256:] == 0xDEADBEEF)
    got = o[16:16 + 256].reshape(64, 4)
    for l in range(64):
        if l < 60:
            np.testing.assert_array_equal(got[l], np.arange(4) + perm[l] * 4)
        else:
            np.testing.assert_array_equal(got[l], 0)


def _mfma_fp8_run(probes, A, B, sa=127, sb=127):
    a = np.zeros((64, 32), np.uint8)
    b = np.zeros((64, 32), np.uint8)
    for l in range(64):
        a[l] = A[l % 32, 32 * (l // 32): 32 * (l // 32) + 32]
        b[l] = B[32 * (l // 32): 32 * (l // 32) + 32, l % 32]
    c = torch.zeros(64, 16, dtype=torch.float32, device="cuda")
    assert probes.probe_mfma_fp8(_p(torch.from_numpy(a).cuda()), _p(torch.from_numpy(b).cuda()), _p(c), sa, sb,
                                 _s()) == 0
    torch.cuda.synchronize()
    cc = c.cpu().numpy()
    got = np.zeros((32, 32))
    for l in range(64):
        for r in range(16):
            got[8 * (r // 4) + 4 * (l // 32) + (r % 4), l % 32] = cc[l, r]
    return got


FP8_ACC_EPS = 2.0 ** -11  # bound on the FP8 product's measured accumulation error (see below)


@pytest.mark.parametrize("codes", ["full_range", "full_range_signed", "block_scaled_gaussian"])
def test_mfma_fp8_accumulation_error(probes, codes):
    """Error of one 64-term FP8 product sum against the exact sum, relative
    to sum |a_k b_k| (the scale of an accumulation error).  The matrix core
    does not keep every bit of a 64-product sum: on codes spanning the whole
    E4M3 range the error reaches about 2^-11.9 of sum |a_k b_k| (2^-12.4
    with random signs), far above fp32 rounding.  This bounds how closely
    FP8 scores of large magnitude can match an exact emulation; recorded
    here, gated at 2^-11."""
    worst = 0.0
    for seed in range(4):
        rng = np.random.default_rng(100 + seed)
        if codes == "block_scaled_gaussian":
            A = e4m3_encode(np.clip(rng.standard_normal((32, 64)) * 112, -448, 448))
            B = e4m3_encode(np.clip(rng.standard_normal((64, 32)) * 112, -448, 448))
        else:
            A = rng.integers(0, 0x7F, size=(32, 64)).astype(np.uint8)
            B = rng.integers(0, 0x7F, size=(64, 32)).astype(np.uint8)
            if codes == "full_range_signed":
                A |= (rng.integers(0, 2, size=A.shape) * 0x80).astype(np.uint8)
                B |= (rng.integers(0, 2, size=B.shape) * 0x80).astype(np.uint8)
        got = _mfma_fp8_run(probes, A, B)
        Ad, Bd = e4m3_decode(A), e4m3_decode(B)
        ref = Ad @ Bd
        mag = np.abs(Ad) @ np.abs(Bd)
        worst = max(worst, float(np.max(np.abs(got - ref) / mag)))
    msg = f"fp8 mfma accumulation error / sum|ab| ({codes}): {worst:.3e} = 2^{np.log2(max(worst, 1e-300)):.2f}"
    print(msg)
    os.makedirs("gpurun_out", exist_ok=True)
    with open("gpurun_out/mfma_accumulation.txt", "a") as f:
        f.write(msg + "\n")
    assert worst <= FP8_ACC_EPS


def test_mfma_bf16_accumulation_error(probes):
    """The same measurement for one 16-term bf16 product sum."""
    worst = 0.0
    for seed in range(4):
        g = torch.Generator().manual_seed(200 + seed)
        A = (torch.randn(32, 16, generator=g) * torch.exp2(torch.randint(-8, 8, (32, 16), generator=g))).to(torch.bfloat16)
        B = (torch.randn(16, 32, generator=g) * torch.exp2(torch.randint(-8, 8, (16, 32), generator=g))).to(torch.bfloat16)
        a = torch.zeros(64, 8, dtype=torch.bfloat16)
        b = torch.zeros(64, 8, dtype=torch.bfloat16)
        for l in range(64):
            a[l] = A[l % 32, 8 * (l // 32): 8 * (l // 32) + 8]
            b[l] = B[8 * (l // 32): 8 * (l // 32) + 8, l % 32]
        c = torch.zeros(64, 16, dtype=torch.float32, device="cuda")
        assert probes.probe_mfma_bf16(_p(a.cuda()), _p(b.cuda()), _p(c), _s()) == 0
        torch.cuda.synchronize()
        cc = c.cpu().numpy()
        got = np.zeros((32, 32))
        for l in range(64):
            for r in range(16):
                got[8 * (r // 4) + 4 * (l // 32) + (r % 4), l % 32] = cc[l, r]
        Ad, Bd = A.double().numpy(), B.double().numpy()
        ref = Ad @ Bd
        mag = np.abs(Ad) @ np.abs(Bd)
        worst = max(worst, float(np.max(np.abs(got - ref) / mag)))
    msg = f"bf16 mfma accumulation error / sum|ab|: {worst:.3e} = 2^{np.log2(max(worst, 1e-300)):.2f}"
    print(msg)
    os.makedirs("gpurun_out", exist_ok=True)
    with open("gpurun_out/mfma_accumulation.txt", "a") as f:
        f.write(msg + "\n")
    assert worst <= 2.0 ** -20
