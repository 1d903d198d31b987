"""FP8 E4M3 emulation: codec, Hadamard rotation, block scales, FP8 attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What the pages fix, and the readings taken where they are silent:

* Format: E4M3 with largest finite magnitude 448 (P2 section 三.3 names
  X_max = 448 for E4M3).  The encoding is the OCP "e4m3fn" one: 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 is
  NaN, subnormals m * 2^-9.  Rounding is to nearest, ties to even, after
  clamping to +-448 (the pages say nothing about rounding or overflow).
* Block quantisation: one scale per block of 128 consecutive rows of one
  (batch, head), all of d (P1 section "Block Quantization 为什么优于
  Per-Tensor Scale" keeps one scale per B_r x d or B_c x d tile; the block
  height of 128 is the plain choice for tiles of 128 query rows).  The scale
  formula was lost from the page text; the plain reading with the 448 bound
  of P2 section 三.3 is s = amax / 448 for each of Q, K and V, and s = 1 for
  an all-zero block.  The code of an entry is the E4M3 rounding of the exact
  quotient y / s (float64 here; no page fixes a precision), so a kernel that
  forms the quotient in fp32 may land one code step away where the exact
  quotient sits within fp32 rounding of a tie.  A power-of-two V scale,
  2^ceil(log2(amax / 448)), is kept as a variant (``pow2``): the matrix
  instruction's E8M0 block exponent carries it exactly and its codes are
  exact in any precision, at the cost of up to one bit of V's range.
  Per-tensor mode uses one amax over the whole tensor (the same section's
  baseline, one scale for all of Q).
* Incoherent processing: Q and K are both multiplied by the same random
  orthogonal matrix M = diag(sigma) H_d / sqrt(d), sigma a per-head vector of
  +-1 and H_d the Sylvester Hadamard matrix (P1 section "Incoherent
  Processing 如何摊平离群值": random +-1 diagonal times Hadamard, so
  (QM)(KM)^T = QK^T in exact arithmetic).  V is not rotated (P1 section
  "为什么 V 不使用同样的 Q/K 成对抵消").
* FP8 attention: S = scale * Q^ K^T on the dequantised operands; both GEMM
  operands are FP8 while the softmax state stays fp32/fp64 (P1 section
  "FP8 Attention 仍然不等于 FP8 全链路"); the V block scale is applied at the
  PV product (P1 section "Block Quantization 为什么优于 Per-Tensor Scale").
  PARITY UNPINNED: the pages never say how the probabilities P = exp(S - m)
  in (0, 1] are brought into FP8.  The reading taken here: write the V
  block's scale as s_V = mu * 2^e with mu in [1, 2); P is quantised as
  P_q = E4M3(P * 2^7 * mu) / (2^7 * mu), so that P * 2^7 * mu < 256 < 448
  never saturates, small probabilities stay out of the subnormal range, and
  the remaining factor 2^e * 2^-7 is an exact power of two.  The row sum l
  is taken from the unquantised P.  The exponent reference of P is the
  running row max rounded up to a whole power of two, M = ln 2 *
  ceil(m / ln 2) (the online-softmax recurrence is exact for any reference
  that bounds the scores seen so far): P = exp(S - M) lies in (0, 1], the
  factors between tiles are exact powers of two, and since E4M3 rounding
  commutes with powers of two in its normal range, P_q * e^M does not depend
  on which whole power is taken except for values in the subnormal range.
  The reading is pinned by a hand-worked two-key case and in the sense that
  with quantisation switched off the emulation equals
  :func:`oracle.attention.attention_ref`.
"""

from __future__ import annotations

import numpy as np

from .attention import to_f64, scale_f64

__all__ = [
    "E4M3_MAX",
    "e4m3_decode",
    "e4m3_encode",
    "e4m3_round",
    "hadamard_matrix",
    "rotation_matrix",
    "quantize_fp8",
    "dequantize_fp8",
    "fp8_attention_emulate",
    "fp8_emulate",
    "scale_mantissa",
    "pow2_ceil",
]

E4M3_MAX = 448.0  # P2 section 三.3
SCALE_BLOCK = 128  # rows per scale block
P_PRESCALE_EXP = 7  # P is scaled by 2^7 * mantissa(s_V) before rounding (parity unpinned)
LN2 = float(np.log(2.0))


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 (e4m3fn) byte, from its bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# the 127 non-negative finite magnitudes, in code order (monotone increasing)
_POS_CODES = np.arange(0, 127, dtype=np.uint8)
_POS_VALS = e4m3_decode(_POS_CODES)


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code, ties to even, after clamping to +-448; NaN -> 0x7F.

    The sign bit is kept for values that round to zero (IEEE-style -0).
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    a_safe = np.where(np.isnan(a), 0.0, a)
    hi = np.searchsorted(_POS_VALS, a_safe, side="left")  # vals[hi-1] < a <= vals[hi]
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a_safe - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a_safe
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a_safe == _POS_VALS[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    code = np.where(neg, code | 0x80, code).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)
    return code


def e4m3_round(x) -> np.ndarray:
    """x rounded to the nearest E4M3 value (clamped), as float64."""
    return e4m3_decode(e4m3_encode(x))


def hadamard_matrix(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_d (entries +-1): H_1 = [1],
    H_2k = [[H_k, H_k], [H_k, -H_k]].  d must be a power of two."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    Hm = np.ones((1, 1), dtype=np.int64)
    while Hm.shape[0] < d:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm


def rotation_matrix(signs) -> np.ndarray:
    """M = diag(sigma) H_d / sqrt(d) for a +-1 vector sigma (orthogonal)."""
    s = np.asarray(signs, dtype=np.float64).reshape(-1)
    d = s.shape[0]
    return (s[:, None] * hadamard_matrix(d)) / np.sqrt(d)


def _rotate_unnormalised(x: np.ndarray, signs) -> np.ndarray:
    """y[b, h] = x[b, h] @ (diag(sigma_h) H_d): the rotation without its
    1/sqrt(d).  For bf16 inputs every entry is a sum of d signed bf16
    values, which float64 holds exactly for the value ranges used here."""
    signs = np.asarray(signs)
    y = np.empty_like(x)
    Hd = hadamard_matrix(x.shape[-1]).astype(np.float64)
    for h in range(x.shape[1]):
        y[:, h] = x[:, h] @ (np.asarray(signs[h], dtype=np.float64)[:, None] * Hd)
    return y


def pow2_ceil(x) -> np.ndarray:
    """Smallest power of two >= x, for positive x (exact: frexp is exact)."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))  # x = m * 2^e, m in [0.5, 1)
    return np.where(m == 0.5, np.ldexp(1.0, e - 1), np.ldexp(1.0, e))


def quantize_fp8(x, signs=None, per_tensor: bool = False, block: int = SCALE_BLOCK, quantize: bool = True,
                 pow2: bool = False):
    """Rotate (optionally), scale and round one tensor ``[B, H, N, d]`` to E4M3.

    With u = x diag(sigma) H_d (unnormalised; u = x without rotation) and
    r = sqrt(d) (1 without rotation), the rotated tensor is y = u / r, the
    block amax is a = max |u| / r and the scale s = a / 448.  The code is
    the E4M3 rounding (nearest, ties to even) of y / s = u * 448 / max|u|,
    taken in float64: u * 448 is exact there and the division rounds once.

    With ``pow2`` (a variant for the PV operand V; no rotation) the scale is
    the power of two s = 2^ceil(log2(a / 448)), the smallest one with
    a / s <= 448, and the code RNE(y / s) is exact in any precision.

    Returns ``(codes, scale, y)``:
      codes uint8 ``[B, H, N, d]`` (None when ``quantize`` is False),
      scale float64 ``[B, H, ceil(N / block)]`` with x_hat = decode(codes) * s,
      y the rotated (or copied) float64 tensor before quantisation.
    """
    x = to_f64(x)
    B, H, N, d = x.shape
    rot = signs is not None
    u = _rotate_unnormalised(x, signs) if rot else x.copy()
    r = np.sqrt(d) if rot else 1.0
    y = u / r
    nb = -(-N // block)
    amax = np.empty((B, H, nb))
    if per_tensor:
        amax[:] = np.abs(u).max() if u.size else 0.0
    else:
        for i in range(nb):
            amax[:, :, i] = np.abs(u[:, :, i * block:(i + 1) * block, :]).max(axis=(2, 3))
    if pow2:
        if rot:
            raise ValueError("power-of-two scales are for the unrotated V operand")
        scale = np.where(amax > 0, pow2_ceil(amax / E4M3_MAX), 1.0)
        if not quantize:
            return None, scale, y
        s_rows = np.repeat(scale, block, axis=2)[:, :, :N, None]
        return e4m3_encode(np.clip(y / s_rows, -E4M3_MAX, E4M3_MAX)), scale, y
    scale = np.where(amax > 0, amax / (E4M3_MAX * r), 1.0)
    if not quantize:
        return None, scale, y
    a_rows = np.repeat(amax, block, axis=2)[:, :, :N, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = np.where(a_rows > 0, (u * E4M3_MAX) / a_rows, 0.0)
    codes = e4m3_encode(np.clip(quot, -E4M3_MAX, E4M3_MAX))
    return codes, scale, y


def dequantize_fp8(codes, scale, block: int = SCALE_BLOCK) -> np.ndarray:
    """decode(codes) * s per 128-row block, float64 ``[B, H, N, d]``."""
    N = codes.shape[2]
    s_rows = np.repeat(np.asarray(scale, dtype=np.float64), block, axis=2)[:, :, :N, None]
    return e4m3_decode(codes) * s_rows


def scale_mantissa(s) -> np.ndarray:
    """mu in [1, 2) with s = mu * 2^e for positive normal s."""
    m, _ = np.frexp(np.asarray(s, dtype=np.float64))
    return 2.0 * m


def fp8_attention_emulate(qh, kh, vh, causal: bool = False, scale=None, Bc: int = 64, quantize_p: bool = True,
                          v_scale=None, block: int = SCALE_BLOCK):
    """Online-softmax attention on already dequantised FP8 operands.

    ``qh, kh, vh`` are float64 ``[B, H, N, d]`` holding exactly the values the
    FP8 codes times their scales represent.  The recurrence is the one of
    :func:`oracle.attention.online_ref` with key blocks of ``Bc`` rows (the
    block size matters here: it decides the running max each probability is
    quantised against; ``Bc`` must divide the scale block).  With
    ``quantize_p`` the PV product uses P_q = E4M3(P * f) / f with
    f = 2^7 * mantissa(s_V) of the key's V scale block (``v_scale``
    ``[B, H, ceil(N / block)]``), while ``l`` sums the unquantised P.  P is
    taken against the running max rounded up to a whole power of two,
    M = ln 2 * ceil(m / ln 2), so P is in (0, 1].
    """
    qh, kh, vh = to_f64(qh), to_f64(kh), to_f64(vh)
    B, H, N, d = qh.shape
    Nk = kh.shape[2]
    if quantize_p:
        if v_scale is None or block % Bc:
            raise ValueError("quantize_p needs v_scale and Bc dividing the scale block")
        fq = np.exp2(P_PRESCALE_EXP) * scale_mantissa(v_scale)  # [B, H, nb]
    sc = scale_f64(scale, d)
    qi = np.arange(N)
    o = np.empty((B, H, N, vh.shape[3]))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            m = np.full(N, -np.inf)  # running max
            r = np.full(N, -np.inf)  # exponent reference: m rounded up to a whole power of two
            l = np.zeros(N)
            acc = np.zeros((N, vh.shape[3]))
            for j0 in range(0, Nk, Bc):
                j1 = min(j0 + Bc, Nk)
                S = sc * (qh[b, h] @ kh[b, h, j0:j1].T)
                if causal:
                    S = np.where(np.arange(j0, j1)[None, :] > qi[:, None], -np.inf, S)
                m_new = np.maximum(m, S.max(axis=1))
                dead = np.isneginf(m_new)
                r_new = np.where(dead, -np.inf, np.ceil(m_new / LN2) * LN2)
                safe = np.where(dead, 0.0, r_new)
                alpha = np.where(dead, 1.0, np.exp(r - safe))
                P = np.where(dead[:, None], 0.0, np.exp(S - safe[:, None]))
                l = alpha * l + P.sum(axis=1)
                if quantize_p:
                    f = fq[b, h, j0 // block]
                    Pq = e4m3_round(P * f) / f
                else:
                    Pq = P
                acc = alpha[:, None] * acc + Pq @ vh[b, h, j0:j1]
                m, r = m_new, r_new
            o[b, h] = acc / l[:, None]
            lse[b, h] = r + np.log(l)
    return o, lse


def fp8_emulate(q, k, v, signs=None, mode: str = "block+had", causal: bool = False, scale=None, Bc: int = 64,
                quantize: bool = True, v_pow2: bool = False):
    """End-to-end FP8 attention emulation in one of three scaling modes.

    mode:
      ``"block+had"`` -- rotate Q and K by diag(signs[h]) H_d / sqrt(d), then
      per-block scales for Q, K and V (the product path);
      ``"block"`` -- per-block scales, no rotation;
      ``"tensor"`` -- one scale per tensor, no rotation (the baseline).
    V's scale is amax / 448 per block (or per tensor), or with ``v_pow2`` the
    power-of-two variant.  With ``quantize=False`` every rounding step is
    skipped, which must give plain attention (the rotation cancels in Q K^T).
    Returns float64 ``(o, lse)``.
    """
    if mode not in ("block+had", "block", "tensor"):
        raise ValueError(mode)
    rot = signs if mode == "block+had" else None
    per_tensor = mode == "tensor"
    out = []
    for x, sg, p2 in ((q, rot, False), (k, rot, False), (v, None, bool(v_pow2))):
        codes, s, y = quantize_fp8(x, signs=sg, per_tensor=per_tensor, quantize=quantize, pow2=p2)
        out.append((dequantize_fp8(codes, s) if quantize else y, s))
    (qh, _), (kh, _), (vh, vs) = out
    return fp8_attention_emulate(qh, kh, vh, causal=causal, scale=scale, Bc=Bc, quantize_p=quantize, v_scale=vs)
