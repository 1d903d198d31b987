"""Pins for oracle/fp8.py: the E4M3 codec, the Hadamard rotation, block and
per-tensor scales, and the FP8 attention emulation."""

import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import (
    E4M3_MAX,
    attention_ref,
    dequantize_fp8,
    e4m3_decode,
    e4m3_encode,
    e4m3_round,
    fp8_attention_emulate,
    fp8_emulate,
    hadamard_matrix,
    quantize_fp8,
    rotation_matrix,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_facts.txt")
RNG = np.random.default_rng(99)


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                rows.append((int(c, 16), float(v)))
    return rows


def test_decode_golden_facts():
    rows = _golden_rows()
    assert (0x7E, E4M3_MAX) in rows
    for c, v in rows:
        got = e4m3_decode(np.uint8(c))
        if math.isnan(v):
            assert np.isnan(got)
        else:
            assert got == v and np.signbit(got) == np.signbit(v)


def test_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(got[fin], ref[fin])
    assert fin.sum() == 254
    pos = got[:127]
    assert np.all(np.diff(pos) > 0) and pos.max() == 448.0 and pos[1] == 2.0 ** -9


def _torch_encode(x):
    t = torch.from_numpy(np.clip(x, -E4M3_MAX, E4M3_MAX)).to(torch.float32)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_dense_sweep_and_ties():
    vals = e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (vals[1:] + vals[:-1]) / 2  # exact ties (representable in float32)
    eps = np.concatenate([mids * (1 - 2.0 ** -20), mids * (1 + 2.0 ** -20)])
    grid = np.linspace(-460, 460, 200001)
    small = np.linspace(-0.02, 0.02, 40001)
    x = np.concatenate([vals, -vals, mids, -mids, eps, -eps, grid, small]).astype(np.float32).astype(np.float64)
    got = e4m3_encode(x)
    ref = _torch_encode(x)
    # compare values (+0 and -0 are the same number)
    np.testing.assert_array_equal(e4m3_decode(got), e4m3_decode(ref))


def test_encode_decode_round_trip_and_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(e4m3_encode(e4m3_decode(codes)), codes)
    assert e4m3_round(1e6) == 448.0 and e4m3_round(-1e6) == -448.0
    assert e4m3_round(2.0 ** -11) == 0.0  # below half the smallest subnormal
    assert e4m3_round(1.0625) == 1.0  # tie between 1.0 and 1.125 goes to even
    assert e4m3_round(1.1875) == 1.25  # tie between 1.125 and 1.25 goes to even
    assert np.isnan(e4m3_round(np.nan))


def test_rounding_error_bound():
    x = RNG.standard_normal(100000) * 50
    x = np.clip(x, -448, 448)
    err = np.abs(e4m3_round(x) - x)
    normal = np.abs(x) >= 2.0 ** -6
    assert np.all(err[normal] <= np.abs(x[normal]) * 2.0 ** -4 + 1e-300)
    assert np.all(err[~normal] <= 2.0 ** -10)


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_is_sylvester_and_orthogonal(d):
    Hm = hadamard_matrix(d)
    np.testing.assert_array_equal(Hm, scipy.linalg.hadamard(d))
    np.testing.assert_array_equal(Hm @ Hm.T, d * np.eye(d, dtype=np.int64))
    s = RNG.choice([-1, 1], d)
    M = rotation_matrix(s)
    np.testing.assert_allclose(M @ M.T, np.eye(d), atol=1e-15)


def test_rotation_preserves_scores_and_attention():
    B, H, N, d = 1, 3, 50, 64
    q, k, v = (RNG.standard_normal((B, H, N, d)) for _ in range(3))
    signs = RNG.choice([-1, 1], (H, d))
    _, _, qr = quantize_fp8(q, signs=signs, quantize=False)
    _, _, kr = quantize_fp8(k, signs=signs, quantize=False)
    for h in range(H):
        np.testing.assert_allclose(qr[0, h] @ kr[0, h].T, q[0, h] @ k[0, h].T, atol=1e-12)
    # the rotation is not the identity: coordinates really change
    assert np.abs(qr - q).max() > 0.1
    o1, l1 = attention_ref(q, k, v)
    o2, l2 = attention_ref(qr, kr, v)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


def test_rotation_spreads_a_channel_outlier():
    d = 128
    x = np.zeros((1, 1, 1, d))
    x[0, 0, 0, 5] = 100.0
    signs = RNG.choice([-1, 1], (1, d))
    _, _, y = quantize_fp8(x, signs=signs, quantize=False)
    np.testing.assert_allclose(np.abs(y), 100.0 / math.sqrt(d), atol=1e-12)


@pytest.mark.parametrize("per_tensor", [False, True])
def test_block_scales_invariants(per_tensor):
    B, H, N, d = 2, 2, 300, 128
    x = RNG.standard_normal((B, H, N, d))
    x[0, 1, 130:140] *= 40  # an outlier region inside block 1
    x[1, 0, 256:] = 0.0  # an all-zero (partial) last block
    signs = None if per_tensor else RNG.choice([-1, 1], (H, d))
    codes, s, y = quantize_fp8(x, signs=signs, per_tensor=per_tensor)
    assert s.shape == (B, H, 3)
    vals = np.abs(e4m3_decode(codes))
    if per_tensor:
        assert np.all(s == s.flat[0]) and vals.max() == 448.0
        np.testing.assert_allclose(s.flat[0], np.abs(x).max() / 448.0, rtol=1e-14)
    else:
        for b in range(B):
            for h in range(H):
                for i in range(3):
                    blk = vals[b, h, i * 128:(i + 1) * 128]
                    if np.abs(y[b, h, i * 128:(i + 1) * 128]).max() == 0:
                        assert s[b, h, i] == 1.0 and blk.max() == 0
                    else:
                        assert blk.max() == 448.0
                        np.testing.assert_allclose(s[b, h, i], np.abs(y[b, h, i * 128:(i + 1) * 128]).max() / 448,
                                                   rtol=1e-14)
    # dequantised values are within half an E4M3 step of y (relative 2^-4)
    xh = dequantize_fp8(codes, s)
    srow = np.repeat(s, 128, axis=2)[:, :, :N, None]
    assert np.all(np.abs(xh - y) <= np.maximum(np.abs(y) * 2.0 ** -4, srow * 2.0 ** -10) + 1e-12)


@pytest.mark.parametrize("Bc", [64, 128])
@pytest.mark.parametrize("mode", ["block+had", "block", "tensor"])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_emulate_without_rounding_is_attention(mode, causal, Bc):
    B, H, N, d = 1, 2, 200, 64
    q, k, v = (RNG.standard_normal((B, H, N, d)) for _ in range(3))
    signs = RNG.choice([-1, 1], (H, d))
    o, l = fp8_emulate(q, k, v, signs=signs, mode=mode, causal=causal, Bc=Bc, quantize=False)
    o_ref, l_ref = attention_ref(q, k, v, causal=causal)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(l, l_ref, atol=1e-12)


def test_fp8_attention_emulate_matches_definition_on_dequantised_operands():
    B, H, N, d = 1, 1, 150, 32
    q, k, v = (RNG.standard_normal((B, H, N, d)) for _ in range(3))
    qh, kh, vh = (dequantize_fp8(*quantize_fp8(x)[:2]) for x in (q, k, v))
    o, l = fp8_attention_emulate(qh, kh, vh, Bc=64, quantize_p=False)
    o_ref, l_ref = attention_ref(qh, kh, vh)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(l, l_ref, atol=1e-12)


def test_fp8_error_is_small_and_ordered_on_outliers():
    # the rounded emulation stays close to exact attention, and per-block
    # scaling with rotation does no worse than one scale per tensor on
    # inputs with large outliers
    B, H, N, d = 1, 2, 512, 128
    g = np.random.default_rng(5)
    q, k, v = (g.standard_normal((B, H, N, d)) for _ in range(3))
    for x in (q, k, v):
        m = g.random(x.shape) < 1e-3
        x[m] = 10 * g.standard_normal(m.sum())
    signs = g.choice([-1, 1], (H, d))
    o_ref, _ = attention_ref(q, k, v)
    rms = {}
    for mode in ("block+had", "block", "tensor"):
        o, _ = fp8_emulate(q, k, v, signs=signs, mode=mode, Bc=64)
        rms[mode] = float(np.sqrt(np.mean((o - o_ref) ** 2)))
    assert rms["block+had"] < 3e-2
    assert rms["block+had"] <= rms["tensor"]


def test_p_quantisation_worked_example():
    """One query, two keys, d = 1, scale 1: scores ln 3 and ln 3 + ln 0.3.
    By hand: the running max ln 3 is log2(3) = 1.58 in base-2 units, so the
    reference is 2^2 and P = (3/4, 0.225); times 2^7: 96 (exact) and 28.8,
    which rounds to 28 on the E4M3 grid (step 2 in [16, 32)).  So P_q =
    (0.75, 0.21875), l = 0.975 from the unrounded P, O = P_q V / l and
    lse = ln(3.9).  (Taking the reference at the exact max instead would give
    P = (1, 0.3) -> 128, 38.4 -> 40 and O = (1, 0.3125) / 1.3.)"""
    qh = np.ones((1, 1, 1, 1))
    kh = np.array([np.log(3.0), np.log(3.0) + np.log(0.3)]).reshape(1, 1, 2, 1)
    vh = np.eye(2).reshape(1, 1, 2, 2)
    o, lse = fp8_attention_emulate(qh, kh, vh, scale=1.0, Bc=2, v_scale=np.ones((1, 1, 1)), block=128)
    np.testing.assert_allclose(o[0, 0, 0], [0.75 / 0.975, 0.21875 / 0.975], rtol=1e-12)
    np.testing.assert_allclose(lse[0, 0, 0], np.log(3.9), rtol=1e-12)


def test_p_quantisation_worked_example_non_power_of_two_v_scale():
    """The two-key case above with s_V = 3 = 1.5 * 2^1 (mu = 1.5): P = (3/4,
    0.225) is brought to FP8 as P * 2^7 * 1.5 = (144, 43.2); 144 is on the
    E4M3 grid and 43.2 rounds to 44 (step 4 in [32, 64)).  So P_q = (144,
    44) / 192, l = 0.975 from the unrounded P, O = P_q V / l, lse = ln(3.9)."""
    qh = np.ones((1, 1, 1, 1))
    kh = np.array([np.log(3.0), np.log(3.0) + np.log(0.3)]).reshape(1, 1, 2, 1)
    vh = np.eye(2).reshape(1, 1, 2, 2)
    o, lse = fp8_attention_emulate(qh, kh, vh, scale=1.0, Bc=2, v_scale=np.full((1, 1, 1), 3.0), block=128)
    np.testing.assert_allclose(o[0, 0, 0], [144 / 192 / 0.975, 44 / 192 / 0.975], rtol=1e-12)
    np.testing.assert_allclose(lse[0, 0, 0], np.log(3.9), rtol=1e-12)


@pytest.mark.parametrize("Bc,pq1", [(1, 0.625 * 2.0 ** -15), (2, 2.0 ** -16)])
def test_p_quantisation_depends_on_the_reference_block(Bc, pq1):
    """Where the reference moves matters only below E4M3's normal range.  One
    query, d = 1, scale 1; scores ln(1.3) - 16 ln 2 and 0, V = I.  With
    blocks of one key the first key's reference is 2^-15 (log2 score -15.62
    rounded up), so P = 0.65, times 2^7 = 83.2, rounds to 80 (step 8 in
    [64, 128)): P_q = 0.625 * 2^-15 once rescaled to the second key's
    reference 2^0.  With one block of both keys the reference is 2^0 from
    the start: P * 2^7 = 1.3 * 2^-9 is subnormal in E4M3 (step 2^-9) and
    rounds to 2^-9, so P_q = 2^-16.  Either way l sums the unrounded P,
    1 + 1.3 * 2^-16, and O = (P_q, 1) / l."""
    qh = np.ones((1, 1, 1, 1))
    kh = np.array([np.log(1.3) - 16 * np.log(2.0), 0.0]).reshape(1, 1, 2, 1)
    vh = np.eye(2).reshape(1, 1, 2, 2)
    o, lse = fp8_attention_emulate(qh, kh, vh, scale=1.0, Bc=Bc, v_scale=np.ones((1, 1, 1)), block=128)
    l = 1 + 1.3 * 2.0 ** -16
    np.testing.assert_allclose(o[0, 0, 0], [pq1 / l, 1 / l], rtol=1e-12)
    np.testing.assert_allclose(lse[0, 0, 0], np.log(l), rtol=1e-12)


def test_fp8_emulate_v_scale_variants():
    """V's default block scale is amax / 448 (every non-zero block reaches
    code 448); the power-of-two variant puts the block amax in (224, 448];
    both emulations stay close to exact attention."""
    g = np.random.default_rng(21)
    B, H, N, d = 1, 2, 256, 64
    q, k, v = (g.standard_normal((B, H, N, d)) for _ in range(3))
    c_v, s_v, _ = quantize_fp8(v)
    for b in range(B):
        for h in range(H):
            for i in range(2):
                assert np.abs(e4m3_decode(c_v[b, h, i * 128:(i + 1) * 128])).max() == 448.0
    mu = s_v / np.exp2(np.floor(np.log2(s_v)))
    assert np.any(mu != 1.0)
    o_ref, _ = attention_ref(q, k, v)
    signs = g.choice([-1, 1], (H, d))
    for v_pow2 in (False, True):
        o, _ = fp8_emulate(q, k, v, signs=signs, Bc=64, v_pow2=v_pow2)
        assert float(np.sqrt(np.mean((o - o_ref) ** 2))) < 2e-2


def test_p_quantisation_invariant_to_the_power_of_two_reference():
    """E4M3 rounding commutes with powers of two in the normal range: shifting
    every score by a whole number of ln 2 moves the reference by the same
    amount and leaves O unchanged (scores here stay far from the subnormal
    range of P)."""
    g = np.random.default_rng(3)
    B, H, N, d = 1, 1, 96, 16
    qh, kh, vh = (g.standard_normal((B, H, N, d)) * 0.3 for _ in range(3))
    vs = np.ones((1, 1, 1))
    o1, l1 = fp8_attention_emulate(qh, kh, vh, scale=1.0, Bc=32, v_scale=vs)
    # add 5 ln 2 to every score via an extra feature: q gets a 1, k gets 5 ln 2
    q2 = np.concatenate([qh, np.ones((B, H, N, 1))], axis=3)
    k2 = np.concatenate([kh, np.full((B, H, N, 1), 5 * np.log(2.0))], axis=3)
    o2, l2 = fp8_attention_emulate(q2, k2, vh, scale=1.0, Bc=32, v_scale=vs)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, l1 + 5 * np.log(2.0), rtol=1e-12)


def test_scale_mantissa_closed_form():
    from oracle import scale_mantissa

    s = np.array([1.0, 3.0, 0.75, 448.0, 2.0 ** -20 * 1.25, 1 / 448])
    mu = scale_mantissa(s)
    np.testing.assert_array_equal(mu, [1.0, 1.5, 1.5, 1.75, 1.25, 2 * 256 / 448])
    e = np.log2(s / mu)
    np.testing.assert_array_equal(e, np.round(e))  # s / mu is an exact power of two


def test_p_quantisation_never_saturates():
    # P in (0, 1] times 2^7 * mu with mu < 2 stays below 256 < 448
    from oracle import scale_mantissa

    mu = scale_mantissa(np.nextafter(2.0, 0))
    assert 2.0 ** 7 * mu < 256 and e4m3_round(2.0 ** 7 * mu) <= 256


def _nearest_e4m3_exact(q):
    """Brute force in exact rational arithmetic: the E4M3 magnitude nearest
    to |q| (ties to the even code), with q clamped to +-448, signed."""
    from fractions import Fraction

    mags = [Fraction(float(v)) for v in e4m3_decode(np.arange(127, dtype=np.uint8))]
    a = min(abs(q), Fraction(448))
    best = min(range(127), key=lambda c: (abs(mags[c] - a), c % 2))
    return -mags[best] if q < 0 else mags[best]


def test_codes_are_the_nearest_e4m3_of_the_exact_quotient():
    """Every code is the E4M3 value nearest to y / s = u * 448 / max|u|,
    checked against brute force over all 127 magnitudes in exact rational
    arithmetic (u and max|u| are exact in float64: sums of bf16 values)."""
    from fractions import Fraction

    g = np.random.default_rng(11)
    x = torch.from_numpy(g.standard_normal((1, 2, 256, 128))).to(torch.bfloat16)
    signs = g.choice([-1, 1], (2, 128))
    for sg in (None, signs):
        codes, s, y = quantize_fp8(x, signs=sg)
        r = np.sqrt(128) if sg is not None else 1.0
        u = y * r  # the unnormalised rotation, exact
        idx = g.integers(0, u.size, 3000)
        for flat in idx:
            b, h, n, c = np.unravel_index(flat, u.shape)
            blk = np.abs(u[b, h, (n // 128) * 128:(n // 128 + 1) * 128]).max()
            q = Fraction(float(u[b, h, n, c])) * 448 / Fraction(float(blk))
            assert Fraction(float(e4m3_decode(codes[b, h, n, c]))) == _nearest_e4m3_exact(q)


def test_codes_at_planted_ties_go_to_even():
    """Block amax 448 (so y / s = y exactly) with entries on E4M3 rounding
    ties: 1.0625 lies between 1 and 1.125 (even: 1), 1.1875 between 1.125
    and 1.25 (even: 1.25), 232 between 224 and 240 (even: 224), and 0.0029296875
    (1.5 * 2^-9) between the subnormals 2^-9 and 2^-8 (even: 2^-8)."""
    x = np.zeros((1, 1, 128, 4))
    x[0, 0, 0, 0] = 448.0
    ties = [1.0625, 1.1875, 232.0, 1.5 * 2.0 ** -9, -1.0625, -232.0]
    want = [1.0, 1.25, 224.0, 2.0 ** -8, -1.0, -224.0]
    for i, t in enumerate(ties):
        x[0, 0, 1 + i, 1] = t
    codes, s, _ = quantize_fp8(x)
    assert s[0, 0, 0] == 1.0
    np.testing.assert_array_equal(e4m3_decode(codes[0, 0, 1:1 + len(ties), 1]), want)


def test_pow2_scale_closed_form():
    from oracle import pow2_ceil

    np.testing.assert_array_equal(pow2_ceil(np.array([1.0, 1.5, 2.0, 3.0, 0.75, 0.5, 2.0 ** -20 * 1.01])),
                                  [1.0, 2.0, 2.0, 4.0, 1.0, 0.5, 2.0 ** -19])


@pytest.mark.parametrize("per_tensor", [False, True])
def test_pow2_block_scales(per_tensor):
    x = RNG.standard_normal((2, 2, 300, 128))
    x[0, 1, 5, 7] = 448.0 * 0.25  # amax exactly 448 * 2^-2 -> s = 2^-2 exactly
    x[1, 0, 256:] = 0.0
    codes, s, y = quantize_fp8(x, per_tensor=per_tensor, pow2=True)
    m, _ = np.frexp(s)
    assert np.all(m == 0.5)  # powers of two
    vals = np.abs(e4m3_decode(codes))
    for b in range(2):
        for h in range(2):
            for i in range(3):
                blk = np.abs(y[b, h, i * 128:(i + 1) * 128]) if not per_tensor else np.abs(y)
                a = blk.max()
                if a == 0:
                    assert s[b, h, i] == 1.0
                    continue
                assert a / s[b, h, i] <= 448 and a / s[b, h, i] > 224
    if not per_tensor:
        assert s[0, 1, 0] == 0.25 and vals[0, 1, 5, 7] == 448.0
    # codes are exact roundings of y / s (a power of two: no rounding before the cast)
    np.testing.assert_array_equal(codes, e4m3_encode(np.clip(y / np.repeat(s, 128, axis=2)[:, :, :300, None], -448, 448)))
    with pytest.raises(ValueError):
        quantize_fp8(x, signs=np.ones((2, 128)), pow2=True)
