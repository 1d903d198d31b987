"""Seeded synthetic inputs: the only code shared by the tests, the oracle
checks and the benchmark.  It holds none of the attention arithmetic.

Recipe (CPU, deterministic; torch's Philox-free CPU generator):

* Q, K, V: ``torch.randn`` float32 ``[B, H, N, d]`` drawn in that order from
  ``torch.Generator("cpu").manual_seed(seed)``, then cast to bfloat16.
* Outlier inputs (the FP8 workload): for each of Q, K, V in that order,
  before the bf16 cast, a mask ``rand < 1e-3`` picks about 0.1 % of the
  entries, which are replaced by ``10 * randn`` (N(0, 10^2)), all drawn from
  the same generator.  The pages' FP8 error study uses a synthetic
  distribution with a few large outliers without giving its parameters.
* Channel-outlier inputs (a second FP8 error report): Q, K, V as above
  (no scattered outliers); then, per head, two channels drawn with
  ``randint(0, d, (H, 2))`` from ``Generator("cpu").manual_seed(seed + 2)``
  are multiplied by 4 in both Q and K before the bf16 cast: outliers that
  sit in the same channel of Q and K, the case the FA3 explainer's section
  on incoherent processing describes.
* Ramped keys (inputs whose row maxima keep growing from key tile to key
  tile): K from any recipe above, row j of n (along the key axis) multiplied
  by 1 + (top - 1) j / (n - 1) in float32, then cast back to bf16.
* Upstream gradient dO (backward): ``torch.randn`` float32 ``[B, H, N, d]``
  from ``Generator("cpu").manual_seed(seed + 2)``, cast to bfloat16.
* Rotation signs: ``[H, d]`` int8 of +-1 from ``randint(0, 2) * 2 - 1`` with
  ``Generator("cpu").manual_seed(seed + 1)``.
* softmax_scale = 1/sqrt(d) as a float32.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = ["make_qkv", "make_qkv_channel_outliers", "ramp_keys", "make_do", "make_signs", "softmax_scale", "Workload",
           "WORKLOADS", "sweep_workloads", "sweep_seed"]


def make_qkv(B: int, H: int, N: int, d: int, seed: int, outliers: bool = False, outlier_frac: float = 1e-3,
             outlier_std: float = 10.0):
    """Return bf16 CPU tensors ``(q, k, v)`` of shape ``[B, H, N, d]``."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    xs = [torch.randn((B, H, N, d), generator=g, dtype=torch.float32) for _ in range(3)]
    if outliers:
        for x in xs:
            m = torch.rand(x.shape, generator=g) < outlier_frac
            x[m] = outlier_std * torch.randn(int(m.sum()), generator=g)
    return tuple(x.to(torch.bfloat16) for x in xs)


def make_qkv_channel_outliers(B: int, H: int, N: int, d: int, seed: int, n_channels: int = 2,
                              factor: float = 4.0):
    """bf16 CPU ``(q, k, v)`` with ``n_channels`` seeded channels per head of
    Q and K multiplied by ``factor`` (the same channels in both)."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    xs = [torch.randn((B, H, N, d), generator=g, dtype=torch.float32) for _ in range(3)]
    gc = torch.Generator("cpu").manual_seed(int(seed) + 2)
    ch = torch.randint(0, d, (H, n_channels), generator=gc)
    for x in xs[:2]:
        for h in range(H):
            x[:, h, :, ch[h]] *= factor
    return tuple(x.to(torch.bfloat16) for x in xs)


def ramp_keys(k: torch.Tensor, top: float, axis: int = 2) -> torch.Tensor:
    """k (bf16) with row j of the key axis scaled by 1 + (top - 1) j / (n - 1)."""
    n = k.shape[axis]
    f = 1.0 + (top - 1.0) * torch.arange(n, dtype=torch.float32) / max(n - 1, 1)
    shape = [1] * k.dim()
    shape[axis] = n
    return (k.float() * f.reshape(shape)).to(torch.bfloat16)


def make_do(B: int, H: int, N: int, d: int, seed: int) -> torch.Tensor:
    """Upstream gradient for the backward: bf16 CPU ``[B, H, N, d]`` drawn from seed + 2."""
    g = torch.Generator("cpu").manual_seed(int(seed) + 2)
    return torch.randn((B, H, N, d), generator=g, dtype=torch.float32).to(torch.bfloat16)


def make_signs(H: int, d: int, seed: int) -> torch.Tensor:
    """Per-head random +-1 vectors, int8 ``[H, d]``."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    return (torch.randint(0, 2, (H, d), generator=g) * 2 - 1).to(torch.int8)


def softmax_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32 (the value passed across the C ABI)."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())


def sweep_seed(N: int, d: int) -> int:
    return 73000 + 100 * (int(math.log2(d)) - 5) + int(math.log2(N))


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: tuple = (False,)
    seed: int = 0
    outliers: bool = False
    fp8: bool = False
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 128, 64, (False,), 73001),
    "std": Workload("std", 4, 16, 2048, 128, (False, True), 73002),
    "long": Workload("long", 1, 16, 65536, 128, (True,), 73400),
    "fp8": Workload("fp8", 4, 16, 4096, 128, (False,), 73500, outliers=True, fp8=True),
}


def packed_batch_lengths(n_seq: int = 16, lo: int = 256, hi: int = 4096, seed: int = 73800) -> list:
    """Sequence lengths of the packed variable-length workload: n_seq seeded
    draws, uniform on [lo, hi] (16 sequences, 36194 tokens by default);
    q is make_qkv(1, H, total, d, seed + 1), k and v make_qkv(..., seed + 2),
    each moved to the token-major [total, H, d] layout."""
    g = torch.Generator("cpu").manual_seed(seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (n_seq,), generator=g)]


def sweep_workloads():
    """Sequence-length sweep at 16384 total tokens and hidden size 2048."""
    out = []
    for d in (64, 128, 256):
        for N in (512, 1024, 2048, 4096, 8192, 16384):
            out.append(Workload(f"sweep_d{d}_N{N}", 16384 // N, 2048 // d, N, d, (False, True), sweep_seed(N, d)))
    return out
