"""Seeded synthetic inputs for the attention workloads.

This module is shared by the GPU path's tests and benchmark and by the float64
oracle's tests.  It only draws random numbers and lays them out; it holds none
of the attention arithmetic.

Recipe (every workload): ``numpy.random.default_rng(seed)`` (PCG64) draws float32
``standard_normal`` arrays in the fixed order Q, K, V, row-major ``[T, H, D]`` for Q
and ``[T, Hkv, D]`` for K and V (seq-major tokens, then heads, then head_dim; Hkv = H
except for grouped-query workloads), then any per-token factors.  bf16
and f16 tensors are the float32 draws rounded to nearest-even by ``torch.Tensor.to``.
The sequence-length prefix array ``cu_seqlens`` is int32 ``[n_seqs + 1]``.

The shapes follow the pages' vision-tower workloads: a 196-patch image at hidden
1152 (16 heads of 72), a 912-patch document page at 16 heads, several images
packed into one call, and a long high-resolution sequence.  The pages measured on
private images with trained weights; these seeded tensors of the same shapes
stand in for them.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = "f32"
BF16 = "bf16"
F16 = "f16"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    lengths: tuple[int, ...]
    n_heads: int
    head_dim: int
    dtype: str
    seed: int
    std: float = 1.0
    token_factor: tuple[float, float] | None = None  # uniform per-token factor on Q and K
    scale: float | None = None  # None -> 1/sqrt(head_dim)
    key_ramp: float = 0.0  # > 0: keys drift along a per-head direction (scores rise or fall along a sequence)
    spikes: int = 0  # keys per sequence pushed far along that direction (a sudden jump of the scores)
    n_kv_heads: int | None = None  # K/V heads (a divisor of n_heads); None -> n_heads

    @property
    def kv_heads(self) -> int:
        return self.n_kv_heads if self.n_kv_heads is not None else self.n_heads

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)

    @property
    def flops(self) -> int:
        """4 * sum_s L_s^2 * D * H: two matmuls of 2*L*L*D flops per head and sequence."""
        return 4 * sum(l * l for l in self.lengths) * self.head_dim * self.n_heads

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)


# The lengths of the packed batch are numpy.random.default_rng(17).integers(256, 4097, 8),
# written out so that the workload does not depend on numpy's stream staying stable.
PACKED_LENGTHS = (3102, 3501, 668, 874, 2015, 2398, 3181, 1669)

WORKLOADS: dict[str, Workload] = {
    "tiny-64": Workload("tiny-64", (64,), 4, 64, F32, seed=1, scale=1.0 / 8.0),
    "vit-196": Workload("vit-196", (196,), 16, 72, BF16, seed=2, std=0.5),
    "page-912": Workload("page-912", (912,), 16, 80, BF16, seed=3, token_factor=(0.5, 2.0)),
    "packed-varlen-8": Workload("packed-varlen-8", PACKED_LENGTHS, 16, 80, BF16, seed=4),
    "long-16384": Workload("long-16384", (16384,), 16, 128, BF16, seed=5),
    # grouped-query attention: the packed batch with 4 K/V heads for the 16 query heads
    "packed-varlen-8-gqa4": Workload("packed-varlen-8-gqa4", PACKED_LENGTHS, 16, 80, BF16, seed=6, n_kv_heads=4),
    # the packed batch in half precision
    "packed-varlen-8-f16": Workload("packed-varlen-8-f16", PACKED_LENGTHS, 16, 80, F16, seed=7),
}


def custom(lengths, n_heads: int, head_dim: int, dtype: str = BF16, seed: int = 0, std: float = 1.0,
           token_factor=None, scale: float | None = None, name: str = "custom", key_ramp: float = 0.0,
           spikes: int = 0, n_kv_heads: int | None = None) -> Workload:
    return Workload(name, tuple(int(x) for x in lengths), int(n_heads), int(head_dim), dtype, int(seed),
                    float(std), token_factor, scale, float(key_ramp), int(spikes),
                    None if n_kv_heads is None else int(n_kv_heads))


def draw_f32(w: Workload) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The float32 draws (before any bf16 rounding): q ``[T, H, D]``, k and v ``[T, Hkv, D]``."""
    rng = np.random.default_rng(w.seed)
    shape = (w.total_tokens, w.n_heads, w.head_dim)
    kv_shape = (w.total_tokens, w.kv_heads, w.head_dim)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(kv_shape, dtype=np.float32)
    v = rng.standard_normal(kv_shape, dtype=np.float32)
    if w.std != 1.0:
        s = np.float32(w.std)
        q *= s
        k *= s
        v *= s
    if w.token_factor is not None:
        lo, hi = w.token_factor
        fq = rng.uniform(lo, hi, size=w.total_tokens).astype(np.float32)
        fk = rng.uniform(lo, hi, size=w.total_tokens).astype(np.float32)
        q *= fq[:, None, None]
        k *= fk[:, None, None]
    if w.key_ramp > 0.0 or w.spikes > 0:
        # direction: random signs per head; key j of a sequence of length L moves by
        # key_ramp * j / L along it, and `spikes` random keys of each sequence by key_ramp more
        sign = np.where(rng.standard_normal((w.kv_heads, w.head_dim)) >= 0, 1.0, -1.0).astype(np.float32)
        cu = w.cu_seqlens()
        for s_ in range(len(w.lengths)):
            a, b = int(cu[s_]), int(cu[s_ + 1])
            if b <= a:
                continue
            pos = (np.arange(b - a, dtype=np.float32) / np.float32(b - a)) * np.float32(w.key_ramp)
            k[a:b] += pos[:, None, None] * sign[None]
            if w.spikes > 0:
                at = rng.integers(a, b, size=w.spikes)
                k[at] += np.float32(w.key_ramp) * sign[None]
    return q, k, v


def make(w: Workload | str):
    """(q, k, v, cu_seqlens, scale) as CPU torch tensors in the workload's dtype."""
    import torch

    if isinstance(w, str):
        w = WORKLOADS[w]
    q, k, v = draw_f32(w)
    tdt = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}[w.dtype]
    qt, kt, vt = (torch.from_numpy(x).to(tdt).contiguous() for x in (q, k, v))
    cu = torch.from_numpy(w.cu_seqlens())
    return qt, kt, vt, cu, w.softmax_scale


def prologue_inputs(lengths, n_heads: int, head_dim: int, dtype: str = BF16, seed: int = 0,
                    n_kv_heads: int | None = None, rope: bool = True, norm: bool = True,
                    theta: float = 100.0):
    """Seeded inputs of the qkv prologue: a dict with ``qkv`` (torch, ``[T, (H + 2*Hkv) * D]``
    in ``dtype``), ``cos``/``sin`` (float32 ``[T, D]`` or None), ``q_weight``/``k_weight``
    (float32 ``[D]`` or None), ``cu_seqlens`` and the head counts.

    Recipe: ``default_rng(seed)`` draws the packed projection output as float32
    ``standard_normal`` (rounded to the 16-bit kinds by torch), then the two gains uniform in
    [0.5, 1.5].  The rope tables follow each image's 2-D patch grid (width ceil(sqrt(L)),
    patch i at row i // width, column i % width): of the D/2 rotated pairs, the first half
    turn with the row and the second half with the column, pair j of a half at frequency
    theta^(-j / (D/4)).  The angle of element d equals that of d + D/2 (the rotate_half
    pairing)."""
    import torch
    hkv = n_heads if n_kv_heads is None else int(n_kv_heads)
    t = int(sum(lengths))
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((t, (n_heads + 2 * hkv) * head_dim), dtype=np.float32)
    qw = rng.uniform(0.5, 1.5, head_dim).astype(np.float32)
    kw = rng.uniform(0.5, 1.5, head_dim).astype(np.float32)
    half, quarter = head_dim // 2, head_dim // 4
    ang = np.zeros((t, half), np.float64)
    pos = 0
    for n in lengths:
        n = int(n)
        if n == 0:
            continue
        width = int(math.ceil(math.sqrt(n)))
        i = np.arange(n)
        r, c = (i // width).astype(np.float64), (i % width).astype(np.float64)
        f_row = theta ** (-np.arange(quarter) / quarter)
        f_col = theta ** (-np.arange(half - quarter) / max(half - quarter, 1))
        ang[pos:pos + n, :quarter] = r[:, None] * f_row[None, :]
        ang[pos:pos + n, quarter:] = c[:, None] * f_col[None, :]
        pos += n
    ang = np.concatenate([ang, ang], axis=1)
    tdt = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}[dtype]
    return {
        "qkv": torch.from_numpy(x).to(tdt),
        "cos": torch.from_numpy(np.cos(ang).astype(np.float32)) if rope else None,
        "sin": torch.from_numpy(np.sin(ang).astype(np.float32)) if rope else None,
        "q_weight": torch.from_numpy(qw) if norm else None,
        "k_weight": torch.from_numpy(kw) if norm else None,
        "cu_seqlens": torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)),
        "n_heads": int(n_heads),
        "n_kv_heads": hkv,
        "head_dim": int(head_dim),
    }
