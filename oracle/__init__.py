"""Float64 CPU oracle for bidirectional multi-head attention over packed sequences.

TEST INFRASTRUCTURE ONLY.  This package is the checker the GPU path is compared
against.  Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it.  It shares no code with the GPU path (the HIP kernels
and their C ABI in ``vision_transformer_attention_amd``) and imports nothing from
it; the seeded input generator is the only module both sides use.

The arithmetic lives in ``vitattn_ref.c`` (plain C, float64, libm ``exp``): for each
sequence ``[cu[s], cu[s+1])``, head ``h`` and query row ``i`` of that sequence,
``O[i,h,:] = sum_j softmax_j(scale * Q[i,h,:].K[j,h,:]) * V[j,h,:]`` with ``j`` over
the same sequence only.  Sources, by page title:

* "inferencelayer 0.2.1 src/vision_gpu.rs" -- vis_attn_coop_src doc, "The obstacle,
  and the way round it" (the online-softmax update whose result is this weighted
  average, and the final division by the row sum); ``VisionGpu::forward_one``
  segment tables (attention stays inside one image; more images are more segments).
* "hf2q src/inference/vision/vit_gpu.rs" -- ``vit_attention_gpu`` doc (no mask, the
  ViT is bidirectional; seq-major ``[tokens, heads, head_dim]``) and
  ``vit_attention_scores_gpu`` doc (the scale is the caller's, 1.0 allowed);
  ``vit_repeat_kv_gpu`` doc and its use in ``gemma4v_block_forward_gpu`` (grouped-query
  attention: K and V carry fewer heads, and query head ``h`` reads K/V head
  ``h // num_kv_groups``).
* "hanzo-ml 0.11.4 src/vulkan_backend.rs" -- ``flash_attn_gpu`` doc (aligned causal
  masking: query ``qi`` sees keys ``kj <= qi + (Lk - Lq)``; inside one image
  ``Lk = Lq``, so ``kj <= qi``).  The key window of the encoder attention meta
  ("inferencelayer 0.2.1 src/vision_gpu.rs", ``VisionGpu::forward_one``: window 0
  is unrestricted) is read as ``|qi - kj| < window``.

``qkv_prologue`` is the input side of the path: the packed projection output split into Q, K and
V, with the optional per-head RMS norm and the rope of "inferencelayer 0.2.1 src/vision_gpu.rs"
(``VIS_QKV_ROPE``, ``GLM_QKV_QKNORM_ROPE``) and the norm definition of "hf2q
src/inference/vision/vit_gpu.rs" (``vit_rms_norm_gpu``: eps inside the square root).

Every function here is pinned by ``tests/test_oracle.py`` against closed forms,
hand-derived golden values, invariants, and a library routine (PyTorch's CPU
``scaled_dot_product_attention`` in float64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vitattn_ref.c")
_LIB_PATH = os.path.join(_HERE, "libvitattn_oracle.so")
_lib = None


def build(out_path: str | None = None, extra_cflags: tuple[str, ...] = ()) -> str:
    """Compile the C oracle with gcc (OpenMP) into a shared library; returns its path."""
    out = out_path or _LIB_PATH
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", *extra_cflags, _SRC, "-lm", "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.vitattn_ref_fwd_f64.argtypes = [f32p, f32p, f32p, f64p, i32p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_double]
    lib.vitattn_ref_fwd_f64.restype = ctypes.c_int
    lib.vitattn_ref_rows_f64.argtypes = [f32p, f32p, f32p, f64p, i32p, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_double, i64p, ctypes.c_int64]
    lib.vitattn_ref_rows_f64.restype = ctypes.c_int
    lib.vitattn_ref_fwd_gqa_f64.argtypes = [f32p, f32p, f32p, f64p, i32p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_double]
    lib.vitattn_ref_fwd_gqa_f64.restype = ctypes.c_int
    lib.vitattn_ref_rows_gqa_f64.argtypes = [f32p, f32p, f32p, f64p, i32p, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_double, i64p, ctypes.c_int64]
    lib.vitattn_ref_rows_gqa_f64.restype = ctypes.c_int
    lib.vitattn_ref_fwd_masked_f64.argtypes = [f32p, f32p, f32p, f64p, i32p, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_int32,
                                               ctypes.c_int32]
    lib.vitattn_ref_fwd_masked_f64.restype = ctypes.c_int
    lib.vitattn_ref_rows_masked_f64.argtypes = [f32p, f32p, f32p, f64p, i32p, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_int32,
                                                ctypes.c_int32, i64p, ctypes.c_int64]
    lib.vitattn_ref_rows_masked_f64.restype = ctypes.c_int
    lib.vitattn_ref_qkv_prologue_f64.argtypes = [f32p, f32p, f32p, f32p, f32p, ctypes.c_double, f64p, f64p, f64p,
                                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.vitattn_ref_qkv_prologue_f64.restype = ctypes.c_int
    lib.vitattn_ref_row_probs_f64.argtypes = [f32p, f32p, i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_double, ctypes.c_int64, ctypes.c_int32, f64p]
    lib.vitattn_ref_row_probs_f64.restype = ctypes.c_int64
    lib.vitattn_ref_threads.argtypes = []
    lib.vitattn_ref_threads.restype = ctypes.c_int
    lib.vitattn_ref_set_threads.argtypes = [ctypes.c_int]
    lib.vitattn_ref_set_threads.restype = None
    return lib


def load(path: str | None = None):
    """Load the compiled oracle (building it first if it is missing)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _as_f32(x) -> np.ndarray:
    """Inputs as contiguous float32 (exact for float32 and bfloat16 data)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().float().numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(np.asarray(x), dtype=np.float32)
    if a.ndim != 3:
        raise ValueError("q/k/v must be [tokens, heads, head_dim]")
    return a


def _cu(cu_seqlens) -> np.ndarray:
    try:
        import torch
        if isinstance(cu_seqlens, torch.Tensor):
            cu_seqlens = cu_seqlens.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int32)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _heads(q, k, v):
    """(T, H, Hkv, D) of q [T, H, D] and k, v [T, Hkv, D], with Hkv a divisor of H."""
    if q.ndim != 3 or k.shape != v.shape or k.ndim != 3:
        raise ValueError("q must be [T, H, D] and k, v the same [T, Hkv, D]")
    t, h, d = q.shape
    if k.shape[0] != t or k.shape[2] != d or k.shape[1] <= 0 or h % k.shape[1] != 0:
        raise ValueError("k and v must be [T, Hkv, D] with Hkv dividing H")
    return t, h, k.shape[1], d


def _mask(causal, window) -> tuple[int, int]:
    if causal not in (False, True, 0, 1) or int(window) < 0:
        raise ValueError("causal must be 0/1 and window >= 0")
    return int(bool(causal)), int(window)


def attention(q, k, v, cu_seqlens, scale: float, lib=None, causal=False, window: int = 0) -> np.ndarray:
    """Full float64 output ``[T, H, D]``; rows outside every sequence stay 0.

    k and v may have fewer heads than q (grouped-query attention): query head h
    uses K/V head h // (H // Hkv).  ``causal`` keeps, inside each sequence, the
    keys at or before the query; ``window`` > 0 keeps the keys less than
    ``window`` positions from it (0: all)."""
    cz, wd = _mask(causal, window)
    lib = lib or load()
    q, k, v = _as_f32(q), _as_f32(k), _as_f32(v)
    cu = _cu(cu_seqlens)
    t, h, hkv, d = _heads(q, k, v)
    if len(cu) < 1 or cu[0] != 0 or cu[-1] != t or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    o = np.zeros((t, h, d), dtype=np.float64)
    rc = lib.vitattn_ref_fwd_masked_f64(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                                        _ptr(v, ctypes.c_float), _ptr(o, ctypes.c_double),
                                        _ptr(cu, ctypes.c_int32), len(cu) - 1, h, hkv, d, float(scale), cz, wd)
    if rc != 0:
        raise RuntimeError("oracle failed")
    return o


def attention_rows(q, k, v, cu_seqlens, scale: float, rows, lib=None, causal=False, window: int = 0) -> np.ndarray:
    """Float64 output for the token rows listed in ``rows`` only: ``[len(rows), H, D]``
    (masks as in ``attention``)."""
    cz, wd = _mask(causal, window)
    lib = lib or load()
    q, k, v = _as_f32(q), _as_f32(k), _as_f32(v)
    cu = _cu(cu_seqlens)
    t, h, hkv, d = _heads(q, k, v)
    if len(cu) < 2 or cu[0] != 0 or cu[-1] != t or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    r = np.ascontiguousarray(np.asarray(rows), dtype=np.int64)
    o = np.zeros((len(r), h, d), dtype=np.float64)
    rc = lib.vitattn_ref_rows_masked_f64(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                                         _ptr(v, ctypes.c_float), _ptr(o, ctypes.c_double),
                                         _ptr(cu, ctypes.c_int32), len(cu) - 1, h, hkv, d, float(scale), cz, wd,
                                         _ptr(r, ctypes.c_int64), len(r))
    if rc != 0:
        raise RuntimeError("oracle failed (bad rows?)")
    return o


def row_probs(q, k, cu_seqlens, scale: float, row: int, head: int, lib=None) -> np.ndarray:
    """The attention weights (float64) of one query row and head over its sequence's keys."""
    lib = lib or load()
    q, k = _as_f32(q), _as_f32(k)
    cu = _cu(cu_seqlens)
    t, h, d = q.shape
    out = np.zeros(max(t, 1), dtype=np.float64)
    n = lib.vitattn_ref_row_probs_f64(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(cu, ctypes.c_int32),
                                      len(cu) - 1, h, d, float(scale), int(row), int(head),
                                      _ptr(out, ctypes.c_double))
    if n < 0:
        raise RuntimeError("oracle failed (bad row/head?)")
    return out[:n].copy()


def _as_f32_any(x, ndim: int) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().float().numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(np.asarray(x), dtype=np.float32)
    if a.ndim != ndim:
        raise ValueError(f"expected {ndim} dimensions, got {a.ndim}")
    return a


def qkv_prologue(qkv, n_heads: int, n_kv_heads: int, cos=None, sin=None, q_weight=None, k_weight=None,
                 eps: float = 1e-6, lib=None):
    """Split a packed projection output ``qkv`` ``[T, (H + 2*Hkv) * D]`` into float64
    ``q [T, H, D]``, ``k [T, Hkv, D]``, ``v [T, Hkv, D]``: Q and K optionally RMS-normalised
    per head (gains ``q_weight``, ``k_weight`` ``[D]``, eps inside the square root) and then
    rotated with the ``cos``/``sin`` tables ``[T, D]`` (rotate_half pairing); V copied."""
    lib = lib or load()
    x = _as_f32_any(qkv, 2)
    t, width = x.shape
    if (cos is None) != (sin is None) or (q_weight is None) != (k_weight is None):
        raise ValueError("give both tables or neither, and both gains or neither")
    if width % (n_heads + 2 * n_kv_heads) != 0:
        raise ValueError("qkv width must be (H + 2*Hkv) * D")
    d = width // (n_heads + 2 * n_kv_heads)
    cs = _as_f32_any(cos, 2) if cos is not None else None
    sn = _as_f32_any(sin, 2) if sin is not None else None
    if cs is not None and (cs.shape != (t, d) or sn.shape != (t, d)):
        raise ValueError("cos and sin must be [T, D]")
    qw = _as_f32_any(q_weight, 1) if q_weight is not None else None
    kw = _as_f32_any(k_weight, 1) if k_weight is not None else None
    if qw is not None and (qw.shape != (d,) or kw.shape != (d,)):
        raise ValueError("gains must be [D]")
    q = np.zeros((t, n_heads, d), np.float64)
    k = np.zeros((t, n_kv_heads, d), np.float64)
    v = np.zeros((t, n_kv_heads, d), np.float64)
    nul = ctypes.POINTER(ctypes.c_float)()
    p = lambda a: _ptr(a, ctypes.c_float) if a is not None else nul
    rc = lib.vitattn_ref_qkv_prologue_f64(_ptr(x, ctypes.c_float), p(cs), p(sn), p(qw), p(kw), float(eps),
                                          _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                          _ptr(v, ctypes.c_double), t, n_heads, n_kv_heads, d)
    if rc != 0:
        raise RuntimeError("oracle prologue failed (bad arguments?)")
    return q, k, v


def threads() -> int:
    """OpenMP threads the oracle's parallel regions use."""
    return int(load().vitattn_ref_threads())


def set_threads(n: int) -> None:
    """Use n OpenMP threads from now on (the results do not depend on it)."""
    load().vitattn_ref_set_threads(int(n))
