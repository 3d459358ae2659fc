"""Thin ctypes binding over ``libvitattn.so`` (argument marshalling only).

Every step of the attention runs in the HIP library; this module checks the
torch tensors' shapes, dtypes, devices and layout, then passes raw device
pointers and the current HIP stream to ``vitattn_fwd`` (or its grouped-query and
masked variants).  There is no fallback:
if the library is missing or the call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libvitattn.so"

DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_F16 = 2
DTYPE_BF16_OUT_F32 = 3
DTYPE_F16_OUT_F32 = 4
HEAD_DIMS = (64, 72, 80, 128)

_lib = None


class VitattnError(RuntimeError):
    """A non-zero status from the HIP library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"vitattn status {status}: {message}")
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def load_library(path: str | None = None):
    """Load ``libvitattn.so`` (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        raise VitattnError(-100, f"{p} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(p)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.vitattn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_float, i32, vp]
    lib.vitattn_fwd.restype = ctypes.c_int
    lib.vitattn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_float, i32, vp]
    lib.vitattn_fwd_gqa.restype = ctypes.c_int
    lib.vitattn_fwd_masked.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_float, i32, i32, i32, vp]
    lib.vitattn_fwd_masked.restype = ctypes.c_int
    f32p = ctypes.c_void_p
    lib.vitattn_qkv_prologue.argtypes = [vp, f32p, f32p, f32p, f32p, ctypes.c_float, vp, vp, vp, i32, i32, i32, i32,
                                         i32, vp]
    lib.vitattn_qkv_prologue.restype = ctypes.c_int
    lib.vitattn_status_string.argtypes = [ctypes.c_int]
    lib.vitattn_status_string.restype = ctypes.c_char_p
    lib.vitattn_last_error.argtypes = []
    lib.vitattn_last_error.restype = ctypes.c_char_p
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.vitattn_kernel_config.argtypes = [i32, i32, i32p, i32p, i32p, i32p]
    lib.vitattn_kernel_config.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _check(lib, status: int) -> None:
    if status != 0:
        detail = lib.vitattn_last_error().decode(errors="replace")
        name = lib.vitattn_status_string(status).decode(errors="replace")
        raise VitattnError(status, f"{name}: {detail}")


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float16:
        return DTYPE_F16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"q/k/v must be bfloat16, float16 or float32, got {t.dtype}")


def _call_code(in_dtype, out_dtype) -> int:
    """The vitattn_dtype_t code for inputs of in_dtype written as out_dtype."""
    import torch
    if out_dtype == in_dtype:
        return {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16}[in_dtype]
    if out_dtype == torch.float32 and in_dtype in (torch.bfloat16, torch.float16):
        return DTYPE_BF16_OUT_F32 if in_dtype == torch.bfloat16 else DTYPE_F16_OUT_F32
    raise TypeError(f"no kernel writes {out_dtype} from {in_dtype} inputs (16-bit inputs may write float32)")


def check_cu_seqlens(cu_host, total_tokens: int) -> None:
    """Host-side check of the cu_seqlens precondition (int32, starts at 0, non-decreasing, ends at T)."""
    import numpy as np
    a = np.asarray(cu_host)
    if a.ndim != 1 or len(a) < 1:
        raise ValueError("cu_seqlens must be a 1-D array of n_seqs + 1 entries")
    if a[0] != 0:
        raise ValueError("cu_seqlens[0] must be 0")
    if np.any(np.diff(a.astype(np.int64)) < 0):
        raise ValueError("cu_seqlens must be non-decreasing")
    if int(a[-1]) != total_tokens:
        raise ValueError(f"cu_seqlens[-1] = {int(a[-1])} must equal the token count {total_tokens}")


def kernel_config(head_dim: int, dtype) -> dict:
    """The launch ``vitattn_fwd`` makes for (head_dim, dtype) on the current device."""
    import torch
    lib = load_library()
    code = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32, torch.float16: DTYPE_F16}.get(dtype, -1)
    vals = [ctypes.c_int32(0) for _ in range(4)]
    _check(lib, lib.vitattn_kernel_config(head_dim, code, *[ctypes.byref(x) for x in vals]))
    return dict(zip(("block_m", "block_n", "waves", "grid"), (x.value for x in vals)))


def fwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, cu_ptr: int, n_seqs: int, n_heads: int,
            head_dim: int, scale: float, dtype_code: int, stream: int) -> None:
    """Direct call of the C entry point with raw pointers (no checks beyond the library's)."""
    lib = load_library()
    _check(lib, lib.vitattn_fwd(q_ptr, k_ptr, v_ptr, o_ptr, cu_ptr, n_seqs, n_heads, head_dim,
                                ctypes.c_float(scale), dtype_code, stream))


def fwd_gqa_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, cu_ptr: int, n_seqs: int, n_heads: int,
                n_kv_heads: int, head_dim: int, scale: float, dtype_code: int, stream: int) -> None:
    """Direct call of the grouped-query C entry point with raw pointers."""
    lib = load_library()
    _check(lib, lib.vitattn_fwd_gqa(q_ptr, k_ptr, v_ptr, o_ptr, cu_ptr, n_seqs, n_heads, n_kv_heads, head_dim,
                                    ctypes.c_float(scale), dtype_code, stream))


def fwd_masked_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, cu_ptr: int, n_seqs: int, n_heads: int,
                   n_kv_heads: int, head_dim: int, scale: float, causal: int, window: int, dtype_code: int,
                   stream: int) -> None:
    """Direct call of the masked C entry point with raw pointers."""
    lib = load_library()
    _check(lib, lib.vitattn_fwd_masked(q_ptr, k_ptr, v_ptr, o_ptr, cu_ptr, n_seqs, n_heads, n_kv_heads, head_dim,
                                       ctypes.c_float(scale), causal, window, dtype_code, stream))


def fwd(q, k, v, cu_seqlens, scale: float | None = None, out=None, check_cu: bool | None = None, out_dtype=None,
        causal: bool = False, window: int = 0):
    """Attention over packed sequences; returns ``o`` like ``q``.

    q: contiguous GPU tensor ``[T, H, D]`` of bfloat16, float16 or float32, D in
    {64, 72, 80, 128}; k, v: the same dtype, ``[T, Hkv, D]`` with Hkv dividing H
    (Hkv < H is grouped-query attention: query head h uses K/V head
    ``h // (H // Hkv)``).  The inputs must be finite (not checked: that would read
    them back): the kernels are built without NaN handling in max/min, and a NaN or
    infinity in q, k or v, or a score that overflows float32, gives unspecified
    output rows for the sequences and heads that read it.  cu_seqlens: int32
    ``[n_seqs + 1]`` prefix array (0, non-decreasing, ending at T).  On q's device it
    is passed to the kernel as it is, and the call neither waits for the device nor
    allocates anything beyond ``out`` (so it can be captured into a HIP graph when
    ``out`` is given); ``check_cu=True`` checks it on the host first, which waits for
    the device.  A CPU tensor is checked on the host (unless ``check_cu=False``) and
    copied to the device.  scale defaults to ``1/sqrt(D)``; any finite value (1.0
    included) is passed through unchanged.  The output has q's dtype, or
    ``out_dtype`` (or ``out``'s dtype): bfloat16 and float16 inputs may be written as
    float32.  By default every query sees every key of its sequence (bidirectional);
    ``causal`` keeps the keys at or before the query and ``window`` > 0 the keys less
    than ``window`` positions from it (both within the sequence).
    """
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device")
        if t.dim() != 3:
            raise ValueError(f"{name} must be [tokens, heads, head_dim]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2] or k.shape[1] <= 0 or q.shape[1] % k.shape[1] != 0:
        raise ValueError("k and v must be [T, Hkv, D] with the tokens and head_dim of q and Hkv dividing q's heads")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k and v must have the same dtype")
    if q.device != k.device or q.device != v.device:
        raise ValueError("q, k and v must be on the same device")
    _dtype_code(q)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else q.dtype
    code = _call_code(q.dtype, out_dtype)
    t_tokens, n_heads, head_dim = q.shape
    if head_dim not in HEAD_DIMS:
        raise ValueError(f"head_dim {head_dim} not in {HEAD_DIMS}")
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise TypeError("cu_seqlens must be a 1-D int32 torch tensor")
    on_device = cu_seqlens.device == q.device
    if check_cu or (check_cu is None and not on_device):
        check_cu_seqlens(cu_seqlens.cpu().numpy(), t_tokens)
    cu_dev = cu_seqlens if on_device else cu_seqlens.to(q.device)
    if not cu_dev.is_contiguous():
        cu_dev = cu_dev.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    if not math.isfinite(scale):
        raise ValueError("scale must be finite")
    if causal not in (False, True, 0, 1):
        raise ValueError("causal must be a bool")
    if int(window) != window or window < 0:
        raise ValueError("window must be an integer >= 0")
    causal, window = int(bool(causal)), int(window)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != out_dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape and device and the output dtype")
    n_seqs = cu_dev.numel() - 1
    if t_tokens == 0 or n_seqs == 0:
        return out
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        n_kv_heads = k.shape[1]
        if causal or window:
            fwd_masked_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), cu_dev.data_ptr(), n_seqs,
                           n_heads, n_kv_heads, head_dim, float(scale), causal, window, code, stream)
        elif n_kv_heads == n_heads:
            fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), cu_dev.data_ptr(), n_seqs, n_heads,
                    head_dim, float(scale), code, stream)
        else:
            fwd_gqa_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), cu_dev.data_ptr(), n_seqs,
                        n_heads, n_kv_heads, head_dim, float(scale), code, stream)
    return out


def qkv_prologue(qkv, n_heads: int, n_kv_heads: int | None = None, cos=None, sin=None, q_weight=None,
                 k_weight=None, eps: float = 1e-6, out=None):
    """Split the packed projection output into the attention inputs; returns ``(q, k, v)``.

    qkv: contiguous GPU tensor ``[T, (H + 2*Hkv) * D]`` (float32, bfloat16 or float16): per token
    the query heads, then the key heads, then the value heads.  ``cos``/``sin``: float32
    ``[T, D]`` rope tables (both or neither); ``q_weight``/``k_weight``: float32 ``[D]`` RMS-norm
    gains (both or neither; eps inside the square root).  Returns ``q [T, H, D]`` and
    ``k, v [T, Hkv, D]`` of qkv's dtype (into ``out`` when given), ready for ``fwd``.
    """
    import torch
    lib = load_library()
    if not isinstance(qkv, torch.Tensor) or qkv.device.type != "cuda" or qkv.dim() != 2 or not qkv.is_contiguous():
        raise ValueError("qkv must be a contiguous 2-D GPU tensor")
    code = _dtype_code(qkv)
    hkv = n_heads if n_kv_heads is None else int(n_kv_heads)
    if n_heads <= 0 or hkv <= 0 or n_heads % hkv != 0:
        raise ValueError("n_kv_heads must be a positive divisor of n_heads")
    t, width = qkv.shape
    if width % (n_heads + 2 * hkv) != 0:
        raise ValueError("qkv width must be (n_heads + 2*n_kv_heads) * head_dim")
    d = width // (n_heads + 2 * hkv)
    if d not in HEAD_DIMS:
        raise ValueError(f"head_dim {d} not in {HEAD_DIMS}")
    if (cos is None) != (sin is None) or (q_weight is None) != (k_weight is None):
        raise ValueError("give both rope tables or neither, and both gains or neither")

    def f32(x, shape, name):
        if x is None:
            return None
        if (not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or x.device != qkv.device
                or tuple(x.shape) != shape or not x.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 tensor of shape {shape} on qkv's device")
        return x
    cos, sin = f32(cos, (t, d), "cos"), f32(sin, (t, d), "sin")
    q_weight, k_weight = f32(q_weight, (d,), "q_weight"), f32(k_weight, (d,), "k_weight")
    if not math.isfinite(eps) or eps < 0:
        raise ValueError("eps must be finite and >= 0")
    if out is None:
        out = (torch.empty((t, n_heads, d), dtype=qkv.dtype, device=qkv.device),
               torch.empty((t, hkv, d), dtype=qkv.dtype, device=qkv.device),
               torch.empty((t, hkv, d), dtype=qkv.dtype, device=qkv.device))
    q, k, v = out
    for x, shape in ((q, (t, n_heads, d)), (k, (t, hkv, d)), (v, (t, hkv, d))):
        if tuple(x.shape) != shape or x.dtype != qkv.dtype or x.device != qkv.device or not x.is_contiguous():
            raise ValueError("out must be contiguous (q, k, v) of the prologue's shapes and qkv's dtype")
    if t == 0:
        return q, k, v
    ptr = lambda x: x.data_ptr() if x is not None else None
    with torch.cuda.device(qkv.device):
        stream = torch.cuda.current_stream(qkv.device).cuda_stream
        _check(lib, lib.vitattn_qkv_prologue(qkv.data_ptr(), ptr(cos), ptr(sin), ptr(q_weight), ptr(k_weight),
                                             ctypes.c_float(eps), q.data_ptr(), k.data_ptr(), v.data_ptr(), t,
                                             n_heads, hkv, d, code, stream))
    return q, k, v
