"""Exact attention (FlashAttention-2 style) forward and backward on AMD MI355X.

A thin ctypes binding over ``libfa2.so``, the C ABI declared in
``include/fa2.h``.  PyTorch only provides device memory and the stream; every
step of the computation runs in the library's HIP kernel.  There is no CPU
fallback: when the library is missing or no GPU is present, calls raise.

    from exact_attention_63_amd import forward
    o, lse = forward(q, k, v, causal=False)        # q, k, v: [B, H, N, d] cuda fp16/bf16
    dq, dk, dv, delta = backward(q, k, v, o, lse, do, causal=False)
    o, lse = forward_fp8(q8, k8, v8, dq, dk, dv)    # E4M3 codes (uint8) and descales
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "forward", "forward_fp8", "fp8_num_variants", "fp8_variant_name", "backward", "bwd_num_variants", "bwd_variant_name", "lib", "lib_path", "status_string", "num_variants", "variant_name", "version",
    "default_variant",
    "FA2_OK", "FA2_ERR_NULL", "FA2_ERR_SHAPE", "FA2_ERR_UNSUPPORTED", "FA2_ERR_ALIGN",
    "FA2_ERR_ARG", "FA2_ERR_ALIAS", "FA2_ERR_LAUNCH", "FA2_DTYPE_FP16", "FA2_DTYPE_BF16",
    "Fa2Error",
]

FA2_OK = 0
FA2_ERR_NULL = -1
FA2_ERR_SHAPE = -2
FA2_ERR_UNSUPPORTED = -3
FA2_ERR_ALIGN = -4
FA2_ERR_ARG = -5
FA2_ERR_ALIAS = -6
FA2_ERR_LAUNCH = -7
FA2_DTYPE_FP16 = 0
FA2_DTYPE_BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfa2.so")
_lib = None

# argument lists of the exported functions (include/fa2.h)
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_FWD12 = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]
EXPORTS = {
    "fa2_fwd_fp16": (_I, _FWD12),
    "fa2_fwd_bf16": (_I, _FWD12),
    "fa2_fwd": (_I, _FWD12 + [_I]),
    "fa2_fwd_variant": (_I, _FWD12 + [_I, _I]),
    "fa2_fwd_check": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I]),
    "fa2_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _F, _F, _P]),
    "fa2_fwd_fp8_check": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _F, _F]),
    "fa2_fwd_fp8_variant": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _F, _F, _P, _I]),
    "fa2_fwd_fp8_variant_check": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _F, _F, _I]),
    "fa2_fp8_num_variants": (_I, []),
    "fa2_fp8_variant_name": (ctypes.c_char_p, [_I]),
    "fa2_fp8_default_variant": (_I, [_I, _I]),
    "fa2_bwd": (_I, [_P] * 10 + [_I, _I, _I, _I, _I, _F, _P, _I]),
    "fa2_bwd_fp16": (_I, [_P] * 10 + [_I, _I, _I, _I, _I, _F, _P]),
    "fa2_bwd_bf16": (_I, [_P] * 10 + [_I, _I, _I, _I, _I, _F, _P]),
    "fa2_bwd_check": (_I, [_P] * 10 + [_I, _I, _I, _I, _I, _F, _I]),
    "fa2_bwd_variant": (_I, [_P] * 10 + [_I, _I, _I, _I, _I, _F, _P, _I, _I]),
    "fa2_bwd_num_variants": (_I, []),
    "fa2_bwd_variant_name": (ctypes.c_char_p, [_I]),
    "fa2_default_variant": (_I, [_I, _I, _I]),
    "fa2_num_variants": (_I, []),
    "fa2_variant_name": (ctypes.c_char_p, [_I]),
    "fa2_status_string": (ctypes.c_char_p, [_I]),
    "fa2_version": (_I, []),
}


class Fa2Error(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libfa2.so (built in-tree by ``python -m exact_attention_63_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m exact_attention_63_amd.build` "
                "(or __graft_entry__.build()); there is no fallback implementation")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().fa2_status_string(status).decode()


def num_variants() -> int:
    return lib().fa2_num_variants()


def variant_name(variant: int) -> str | None:
    s = lib().fa2_variant_name(variant)
    return None if s is None else s.decode()


def default_variant(dtype, d: int, causal: bool) -> int:
    """The tile variant that variant 0 resolves to (dtype: torch dtype or FA2_DTYPE_*)."""
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    rc = lib().fa2_default_variant(code, d, int(bool(causal)))
    if rc < 0:
        raise Fa2Error(rc, "fa2_default_variant")
    return rc


def version() -> int:
    return lib().fa2_version()


def _dtype_code(dtype) -> int:
    import torch
    if dtype == torch.float16:
        return FA2_DTYPE_FP16
    if dtype == torch.bfloat16:
        return FA2_DTYPE_BF16
    raise ValueError(f"q, k, v must be float16 or bfloat16, got {dtype}")


def _check_empty(d: int, variant: int, nvar: int) -> None:
    """The library's argument checks that still apply to an empty problem."""
    if not 0 <= int(variant) < nvar:
        raise Fa2Error(FA2_ERR_ARG, "variant")
    if d not in (64, 128):
        raise Fa2Error(FA2_ERR_UNSUPPORTED, "head dimension")


def forward(q, k, v, causal: bool = False, scale: float | None = None, *, variant: int = 0,
            out=None, lse=None):
    """Attention forward: returns (O [B,H,N,d] in q's dtype, LSE [B,H,N] float32).

    q, k, v: contiguous CUDA (ROCm) tensors [B, H, N, d] of one dtype (fp16 or
    bf16), d in {64, 128}.  scale defaults to 1/sqrt(d).  The kernel is
    enqueued on the current stream of q's device; the call does not
    synchronise.  ``out`` / ``lse`` may pass preallocated outputs.  An empty
    problem (B, H or N == 0) returns the empty outputs without a library call
    (the C ABI returns FA2_ERR_SHAPE for it).
    """
    import torch
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share one shape [B, H, N, d]; got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    code = _dtype_code(q.dtype)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != q.device:
            raise ValueError("q, k, v must be on one device")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor [B, H, N] on q's device")
    if out.numel() == 0:
        # B, H or N is 0: nothing to compute (the library rejects empty sizes)
        _check_empty(d, variant, num_variants())
        return out, lse
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        rc = lib().fa2_fwd_variant(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, H, N, d, int(bool(causal)), float(scale),
                                   stream, code, int(variant))
    if rc != FA2_OK:
        raise Fa2Error(rc, "fa2_fwd_variant")
    return out, lse


def forward_fp8(q, k, v, descale_q: float, descale_k: float, descale_v: float, causal: bool = False,
                scale: float | None = None, *, out=None, lse=None, variant: int = 0):
    """FP8 attention forward: returns (O [B,H,N,d] bfloat16, LSE [B,H,N] float32).

    q, k, v: contiguous CUDA (ROCm) uint8 tensors [B, H, N, d] of OCP E4M3
    codes (a float8_e4m3fn tensor viewed as uint8), d in {64, 128}; the
    inputs are decode(q) * descale_q etc.  scale defaults to 1/sqrt(d).
    variant 0 calls fa2_fwd_fp8; any other calls fa2_fwd_fp8_variant.
    Enqueued on the current stream of q's device; the call does not
    synchronise.  An empty problem returns the empty outputs without a
    library call.
    """
    import torch
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share one shape [B, H, N, d]; got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.uint8:
            raise ValueError(f"{name} must hold E4M3 codes as uint8, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != q.device:
            raise ValueError("q, k, v must be on one device")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor [B, H, N] on q's device")
    if out.numel() == 0:
        if d not in (64, 128):
            raise Fa2Error(FA2_ERR_UNSUPPORTED, "head dimension")
        return out, lse
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                int(bool(causal)), float(scale), float(descale_q), float(descale_k), float(descale_v), stream)
        if variant == 0:
            rc, where = lib().fa2_fwd_fp8(*args), "fa2_fwd_fp8"
        else:
            rc, where = lib().fa2_fwd_fp8_variant(*args, int(variant)), "fa2_fwd_fp8_variant"
    if rc != FA2_OK:
        raise Fa2Error(rc, where)
    return out, lse


def fp8_num_variants() -> int:
    return lib().fa2_fp8_num_variants()


def fp8_variant_name(variant: int) -> str | None:
    name = lib().fa2_fp8_variant_name(variant)
    return None if name is None else name.decode()


def bwd_num_variants() -> int:
    return lib().fa2_bwd_num_variants()


def bwd_variant_name(variant: int) -> str | None:
    s = lib().fa2_bwd_variant_name(variant)
    return None if s is None else s.decode()


def backward(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None, *,
             variant: int = 0, dq=None, dk=None, dv=None, delta=None):
    """Attention backward: returns (dQ, dK, dV in q's dtype, delta [B,H,N] float32).

    q, k, v, o, do: contiguous CUDA tensors [B, H, N, d] of one dtype (fp16 or
    bf16), d in {64, 128}; o and lse [B, H, N] float32 are the forward pass's
    outputs for q, k, v with the same causal flag and scale (default
    1/sqrt(d)).  delta receives rowsum(dO * O).  The three kernels are
    enqueued on the current stream of q's device; the call does not
    synchronise.  dq, dk, dv, delta may pass preallocated outputs.  variant
    selects the dK/dV kernel configuration (0 = default, see
    ``bwd_variant_name``).
    """
    import torch
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H, N, d]; got {tuple(q.shape)}")
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        if t.shape != q.shape:
            raise ValueError(f"{name} must have q's shape {tuple(q.shape)}; got {tuple(t.shape)}")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} must have q's dtype")
    code = _dtype_code(q.dtype)
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 tensor [B, H, N]")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("do", do)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor like q")
    if delta.shape != (B, H, N) or delta.dtype != torch.float32 or not delta.is_contiguous() \
            or delta.device != q.device:
        raise ValueError("delta must be a contiguous float32 tensor [B, H, N] on q's device")
    if dq.numel() == 0:
        _check_empty(d, variant, bwd_num_variants())
        return dq, dk, dv, delta
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        rc = lib().fa2_bwd_variant(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                   delta.data_ptr(), B, H, N, d, int(bool(causal)), float(scale), stream,
                                   code, int(variant))
    if rc != FA2_OK:
        raise Fa2Error(rc, "fa2_bwd_variant")
    return dq, dk, dv, delta
