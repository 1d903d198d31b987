"""ctypes binding of the C ABI in include/fa.h (argument marshalling only).

Every step of the attention path runs in the HIP kernels of ``libfa.so``;
this module only checks tensor metadata, allocates outputs with torch,
passes raw device pointers and the current stream, and turns a non-zero
status into an exception.  There is no other implementation to fall back
to: if the library is missing or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_NAME = "libfa.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

FA_PREP_TRANSPOSE = 1
FA_PREP_PER_TENSOR = 2
FA_PREP_POW2_SCALE = 4

# every function the header declares, with its ctypes signature
_VP, _FP, _I, _F, _LL = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_longlong
SIGNATURES = {
    "fa_fwd_bf16": (_I, [_VP, _VP, _VP, _FP, _FP, _I, _I, _I, _I, _I, _F, _VP]),
    "fa_fwd_bf16_gqa": (_I, [_VP, _VP, _VP, _FP, _FP, _I, _I, _I, _I, _I, _I, _I, _F, _VP]),
    "fa_fwd_bf16_varlen": (_I, [_VP, _VP, _VP, _FP, _FP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _I, _F, _VP]),
    "fa_fwd_bf16_decode_splits": (_I, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "fa_fwd_bf16_decode_workspace": (_LL, [_I, _I, _I, _I, _I]),
    "fa_fwd_bf16_decode": (_I, [_VP, _VP, _VP, _FP, _FP, _I, _I, _I, _I, _I, _I, _I, _F, _I, _VP, _LL, _VP]),
    "fa_fwd_bf16_decode_noalloc": (_I, [_VP, _VP, _VP, _FP, _FP, _I, _I, _I, _I, _I, _I, _I, _F, _I, _VP]),
    "fa_bwd_bf16_gqa": (_I, [_VP, _VP, _VP, _FP, _FP, _VP, _FP, _FP, _FP, _FP, _I, _I, _I, _I, _I, _I, _F, _VP]),
    "fa_bwd_bf16": (_I, [_VP, _VP, _VP, _FP, _FP, _VP, _FP, _FP, _FP, _FP, _I, _I, _I, _I, _I, _F, _VP]),
    "fa_fp8_prep": (_I, [_VP, _VP, _FP, _VP, _I, _I, _I, _I, ctypes.c_uint, _VP]),
    "fa_fp8_vt_ld": (_I, [_I]),
    "fa_fp8_ref_block": (_I, [_I, _I]),
    "fa_fwd_fp8": (_I, [_VP, _VP, _VP, _FP, _FP, _FP, _FP, _FP, _I, _I, _I, _I, _I, _F, _VP]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_abi_version": (_I, []),
}

_lib = None


class FaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library once; raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run __graft_entry__.build() (hipcc for gfx950) first")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise FaError(fn, status, load().fa_status_string(status).decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor on a GPU")


def _out(t, shape, dtype, device, name):
    """A new output tensor, or the caller's after checking dtype, device,
    contiguity and shape (a short buffer would be an out-of-bounds write)."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def fwd_bf16(q, k, v, causal: bool = False, softmax_scale: float | None = None, out=None, lse=None):
    """O, lse = attention(q, k, v) for bf16 ``[B, H, N, d]`` CUDA tensors.

    Returns fp32 ``o [B, H, N, d]`` and fp32 ``lse [B, H, N]`` (natural log).
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, n)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one shape [B, H, N, d]")
    B, H, N, d = q.shape
    scale = (1.0 / d ** 0.5) if softmax_scale is None else float(softmax_scale)
    o = _out(out, (B, H, N, d), torch.float32, q.device, "out")
    ls = _out(lse, (B, H, N), torch.float32, q.device, "lse")
    st = load().fa_fwd_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), ls.data_ptr(), B, H, N, d,
                            int(bool(causal)), scale, _stream(q))
    _check("fa_fwd_bf16", st)
    return o, ls


def fp8_vt_ld(N: int) -> int:
    return int(load().fa_fp8_vt_ld(int(N)))


def fp8_ref_block(N: int, causal: bool = False) -> int:
    """Keys per exponent-reference step of :func:`fwd_fp8` for ``N`` keys."""
    r = int(load().fa_fp8_ref_block(int(N), int(bool(causal))))
    _check("fa_fp8_ref_block", r if r < 0 else 0)
    return r


def fwd_bf16_gqa(q, k, v, causal: bool = False, softmax_scale: float | None = None, out=None, lse=None):
    """Forward for q ``[B, Hq, Nq, d]`` and k, v ``[B, Hkv, Nk, d]`` (bf16);
    bottom-right causal alignment. Returns fp32 ``o [B, Hq, Nq, d]``, ``lse [B, Hq, Nq]``."""
    B, Hq, Hkv, Nq, Nk, d = _gqa_shapes(q, k, v)
    scale = (1.0 / d ** 0.5) if softmax_scale is None else float(softmax_scale)
    o = _out(out, (B, Hq, Nq, d), torch.float32, q.device, "out")
    ls = _out(lse, (B, Hq, Nq), torch.float32, q.device, "lse")
    st = load().fa_fwd_bf16_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), ls.data_ptr(), B, Hq, Hkv,
                                Nq, Nk, d, int(bool(causal)), scale, _stream(q))
    _check("fa_fwd_bf16_gqa", st)
    return o, ls


def _gqa_shapes(q, k, v):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, n)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError("q must be [B, Hq, Nq, d] and k, v [B, Hkv, Nk, d]")
    B, Hq, Nq, d = q.shape
    return B, Hq, k.shape[1], Nq, k.shape[2], d


def fwd_bf16_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, causal: bool = False,
                    softmax_scale: float | None = None, out=None, lse=None):
    """Forward over packed sequences: q ``[total_q, Hq, d]``, k, v
    ``[total_k, Hkv, d]`` (bf16), ``cu_seqlens_*`` int32 ``[B + 1]`` on the
    GPU.  Returns fp32 ``o [total_q, Hq, d]`` and ``lse [Hq, total_q]``."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, n)
    _need(cu_seqlens_q, torch.int32, "cu_seqlens_q")
    _need(cu_seqlens_k, torch.int32, "cu_seqlens_k")
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or k.shape[2] != q.shape[2]:
        raise ValueError("q must be [total_q, Hq, d] and k, v [total_k, Hkv, d]")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_k.shape != cu_seqlens_q.shape or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be [B + 1]")
    total_q, Hq, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.numel() - 1
    scale = (1.0 / d ** 0.5) if softmax_scale is None else float(softmax_scale)
    o = _out(out, (total_q, Hq, d), torch.float32, q.device, "out")
    ls = _out(lse, (Hq, total_q), torch.float32, q.device, "lse")
    st = load().fa_fwd_bf16_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), ls.data_ptr(),
                                   cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, Hq, Hkv, total_q, total_k,
                                   int(max_seqlen_q), d, int(bool(causal)), scale, _stream(q))
    _check("fa_fwd_bf16_varlen", st)
    return o, ls


def decode_splits(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, num_splits: int = 0,
                  num_cus: int | None = None) -> int:
    """Key chunks per KV head that ``fwd_bf16_decode`` uses (0 = the cost
    model's choice for ``num_cus`` compute units, default: the current GPU's)."""
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    s = load().fa_fwd_bf16_decode_splits(B, Hq, Hkv, Nq, Nk, d, int(num_splits), int(num_cus))
    if s < 0:
        _check("fa_fwd_bf16_decode_splits", s)
    return s


def decode_workspace_bytes(B: int, Hq: int, Nq: int, d: int, splits: int) -> int:
    n = load().fa_fwd_bf16_decode_workspace(B, Hq, Nq, d, splits)
    if n < 0:
        _check("fa_fwd_bf16_decode_workspace", int(n))
    return int(n)


def fwd_bf16_decode(q, k, v, causal: bool = False, softmax_scale: float | None = None, num_splits: int = 0,
                    out=None, lse=None, workspace=None):
    """Split-KV forward for few queries against long keys: q ``[B, Hq, Nq, d]``,
    k, v ``[B, Hkv, Nk, d]`` (bf16); same result as ``fwd_bf16_gqa``.
    ``num_splits`` 0 lets the library choose; ``workspace`` (any dtype,
    contiguous, on the GPU) is allocated when omitted and needed."""
    B, Hq, Hkv, Nq, Nk, d = _gqa_shapes(q, k, v)
    scale = (1.0 / d ** 0.5) if softmax_scale is None else float(softmax_scale)
    cus = torch.cuda.get_device_properties(q.device).multi_processor_count
    splits = decode_splits(B, Hq, Hkv, Nq, Nk, d, num_splits, cus)
    need = decode_workspace_bytes(B, Hq, Nq, d, splits)
    if need > 0 and workspace is None:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on a GPU")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    o = _out(out, (B, Hq, Nq, d), torch.float32, q.device, "out")
    ls = _out(lse, (B, Hq, Nq), torch.float32, q.device, "lse")
    st = load().fa_fwd_bf16_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), ls.data_ptr(), B, Hq,
                                   Hkv, Nq, Nk, d, int(bool(causal)), scale, splits, ws_ptr, ws_bytes, _stream(q))
    _check("fa_fwd_bf16_decode", st)
    return o, ls


def fwd_bf16_decode_noalloc(q, k, v, causal: bool = False, softmax_scale: float | None = None, num_splits: int = 0,
                            out=None, lse=None):
    """``fwd_bf16_decode`` without a workspace: the chunk partials go to the
    library's static per-device scratch buffer (16 MiB), so the call itself
    allocates no device memory (pass ``out`` and ``lse`` for that).
    ``num_splits`` 0 lets the library choose a count whose partials fit;
    calls that overlap in time on one device race on the shared buffer."""
    B, Hq, Hkv, Nq, Nk, d = _gqa_shapes(q, k, v)
    scale = (1.0 / d ** 0.5) if softmax_scale is None else float(softmax_scale)
    o = _out(out, (B, Hq, Nq, d), torch.float32, q.device, "out")
    ls = _out(lse, (B, Hq, Nq), torch.float32, q.device, "lse")
    st = load().fa_fwd_bf16_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), ls.data_ptr(), B,
                                           Hq, Hkv, Nq, Nk, d, int(bool(causal)), scale, int(num_splits), _stream(q))
    _check("fa_fwd_bf16_decode_noalloc", st)
    return o, ls


def bwd_bf16(q, k, v, o, lse, dout, causal: bool = False, softmax_scale: float | None = None, dq=None, dk=None,
             dv=None, delta=None):
    """dQ, dK, dV (fp32 ``[B, H, N, d]``) of the forward for the upstream
    gradient ``dout`` (bf16), from the forward's ``o`` and ``lse`` (fp32).
    ``delta`` is the fp32 ``[B, H, N]`` workspace (allocated when omitted)."""
    return _bwd("fa_bwd_bf16", q, k, v, o, lse, dout, causal, softmax_scale, dq, dk, dv, delta)


def bwd_bf16_gqa(q, k, v, o, lse, dout, causal: bool = False, softmax_scale: float | None = None, dq=None, dk=None,
                 dv=None, delta=None):
    """Backward with grouped/multi-query heads: q, dout, o ``[B, Hq, N, d]``,
    k, v ``[B, Hkv, N, d]``; returns fp32 dq ``[B, Hq, N, d]`` and dk, dv
    ``[B, Hkv, N, d]`` (each KV head's gradient summed over its query heads)."""
    return _bwd("fa_bwd_bf16_gqa", q, k, v, o, lse, dout, causal, softmax_scale, dq, dk, dv, delta)


def _bwd(fn, q, k, v, o, lse, dout, causal, softmax_scale, dq, dk, dv, delta):
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _need(t, torch.bfloat16, n)
    _need(o, torch.float32, "o")
    _need(lse, torch.float32, "lse")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or any(t.shape != q.shape for t in (dout, o)):
        raise ValueError("q, dout, o must be [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError("k, v must be [B, Hkv, N, d] with the queries' B, N, d")
    if fn == "fa_bwd_bf16" and Hkv != H:
        raise ValueError("q, k, v, dout, o must share one shape [B, H, N, d] (use bwd_bf16_gqa for grouped heads)")
    if tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be [B, H, N]")
    scale = (1.0 / d ** 0.5) if softmax_scale is None else float(softmax_scale)
    outs = []
    for t, n, h in ((dq, "dq", H), (dk, "dk", Hkv), (dv, "dv", Hkv)):
        t = torch.empty((B, h, N, d), dtype=torch.float32, device=q.device) if t is None else t
        _need(t, torch.float32, n)
        if tuple(t.shape) != (B, h, N, d):
            raise ValueError(f"{n} must be [B, {h}, N, d]")
        outs.append(t)
    ws = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if delta is None else delta
    _need(ws, torch.float32, "delta")
    if tuple(ws.shape) != (B, H, N):
        raise ValueError("delta must be [B, H, N]")
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
            outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), ws.data_ptr())
    lib = load()
    if fn == "fa_bwd_bf16":
        st = lib.fa_bwd_bf16(*ptrs, B, H, N, d, int(bool(causal)), scale, _stream(q))
    else:
        st = lib.fa_bwd_bf16_gqa(*ptrs, B, H, Hkv, N, d, int(bool(causal)), scale, _stream(q))
    _check(fn, st)
    return tuple(outs)


def fp8_prep(x, signs=None, transpose: bool = False, per_tensor: bool = False, pow2_scale: bool = False,
             out=None, scale_out=None):
    """E4M3 codes and per-128-row scales of one bf16 ``[B, H, N, d]`` tensor.

    ``signs``: int8 ``[H, d]`` of +-1 on the GPU (rotate, for Q and K) or None.
    For V use ``transpose=True`` without signs (:func:`fp8_prep_v`).
    Returns ``(x8, scale)``: uint8 ``[B, H, N, d]`` (or ``[B, H, d, ld]`` when
    ``transpose``) and fp32 ``[B, H, ceil(N / 128)]``, written into ``out`` and
    ``scale_out`` when given.
    """
    _need(x, torch.bfloat16, "x")
    B, H, N, d = x.shape
    if signs is not None:
        _need(signs, torch.int8, "signs")
        if tuple(signs.shape) != (H, d):
            raise ValueError("signs must be [H, d]")
    nb = (N + 127) // 128
    shape = (B, H, d, fp8_vt_ld(N)) if transpose else (B, H, N, d)
    x8 = torch.empty(shape, dtype=torch.uint8, device=x.device) if out is None else out
    sc = torch.empty((B, H, nb), dtype=torch.float32, device=x.device) if scale_out is None else scale_out
    _need(x8, torch.uint8, "out")
    _need(sc, torch.float32, "scale_out")
    if tuple(x8.shape) != shape or tuple(sc.shape) != (B, H, nb):
        raise ValueError(f"out must be {shape} and scale_out {(B, H, nb)}")
    flags = ((FA_PREP_TRANSPOSE if transpose else 0) | (FA_PREP_PER_TENSOR if per_tensor else 0)
             | (FA_PREP_POW2_SCALE if pow2_scale else 0))
    st = load().fa_fp8_prep(x.data_ptr(), x8.data_ptr(), sc.data_ptr(), None if signs is None else signs.data_ptr(),
                            B, H, N, d, flags, _stream(x))
    _check("fa_fp8_prep", st)
    return x8, sc


def fp8_prep_v(v, per_tensor: bool = False, pow2_scale: bool = False, out=None, scale_out=None):
    """The PV operand: V transposed, never rotated, with block (or tensor)
    scales amax / 448, or with ``pow2_scale`` the power-of-two variant
    2^ceil(log2(amax / 448))."""
    return fp8_prep(v, transpose=True, per_tensor=per_tensor, pow2_scale=pow2_scale, out=out, scale_out=scale_out)


def fwd_fp8(q8, k8, v8t, q_scale, k_scale, v_scale, causal: bool = False, softmax_scale: float | None = None,
            out=None, lse=None):
    """Attention forward on the FP8 operands made by :func:`fp8_prep`."""
    for t, n in ((q8, "q8"), (k8, "k8"), (v8t, "v8t")):
        _need(t, torch.uint8, n)
    for t, n in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        _need(t, torch.float32, n)
    B, H, N, d = q8.shape
    if k8.shape != q8.shape or tuple(v8t.shape) != (B, H, d, fp8_vt_ld(N)):
        raise ValueError("k8 must match q8 and v8t must be [B, H, d, fa_fp8_vt_ld(N)]")
    nb = (N + 127) // 128
    for t in (q_scale, k_scale, v_scale):
        if tuple(t.shape) != (B, H, nb):
            raise ValueError("scales must be [B, H, ceil(N / 128)]")
    scale = (1.0 / d ** 0.5) if softmax_scale is None else float(softmax_scale)
    o = _out(out, (B, H, N, d), torch.float32, q8.device, "out")
    ls = _out(lse, (B, H, N), torch.float32, q8.device, "lse")
    st = load().fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8t.data_ptr(), q_scale.data_ptr(), k_scale.data_ptr(),
                           v_scale.data_ptr(), o.data_ptr(), ls.data_ptr(), B, H, N, d, int(bool(causal)), scale,
                           _stream(q8))
    _check("fa_fwd_fp8", st)
    return o, ls
