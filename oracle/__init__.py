"""CPU fp64 oracle for the fused exact attention forward and its FP8 variant.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, calls or links anything here.  The only callers
are the tests under ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The oracle shares no code, tables or
constants with the GPU path; both sides only share the seeded input
generators, which hold none of the method's arithmetic.

Pages cited (all are web pages about FlashAttention-3):

* [P1] "FlashAttention-3：用异步流水榨出 Hopper 的 Attention 性能"
  (charlestar.github.io, 2026-06-23), cited by section heading.
* [P2] FlashAttention V3 article on wmrh.cn (news/71740), cited by its
  numbered sections (e.g. "一.1", "二.1", "三.3").
* [P3] "FlashAttention-3" encyclopedia entry (newton.com.tw).
* [P4] Flash Attention V3 async article (aiqz.cc).

Modules:

* :mod:`oracle.attention` -- ``attention_ref`` (the plain definition, S
  materialised) and ``online_ref`` (the tiled online-softmax recurrence).
* :mod:`oracle.gqa` -- ``attention_gqa_ref`` (grouped/multi-query heads,
  unequal query and key lengths, bottom-right causal alignment).
* :mod:`oracle.varlen` -- ``attention_varlen_ref`` (sequences of different
  lengths packed end to end, token-major layout).
* :mod:`oracle.backward` -- ``attention_bwd_ref`` (dQ, dK, dV of the
  definition, written out) and ``attention_gqa_bwd_ref`` (grouped heads:
  each KV head's gradient summed over the query heads that read it).
* :mod:`oracle.fp8` -- OCP E4M3 codec, Sylvester Hadamard rotation, per-block
  and per-tensor scaling, and ``fp8_attention_emulate``.

Every function is pinned by ``-m "not gpu"`` tests against facts that do not
come from the oracle itself (brute force, closed forms, library routines,
invariants).  The one reading that nothing on the pages fixes -- how
probabilities are scaled before their E4M3 cast in the FP8 PV product -- is
marked "parity unpinned" in :mod:`oracle.fp8`.
"""

from .attention import attention_ref, online_ref  # noqa: F401
from .backward import attention_bwd_ref, attention_gqa_bwd_ref  # noqa: F401
from .gqa import attention_gqa_ref  # noqa: F401
from .varlen import attention_varlen_ref  # noqa: F401
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    e4m3_round,
    hadamard_matrix,
    rotation_matrix,
    quantize_fp8,
    dequantize_fp8,
    fp8_attention_emulate,
    fp8_emulate,
    scale_mantissa,
    pow2_ceil,
)
