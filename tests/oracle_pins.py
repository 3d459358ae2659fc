"""Checks that pin the float64 oracle to facts other than itself.

Each check takes the loaded oracle library and raises AssertionError on a miss.
They are closed forms worked out by hand (``golden/closed_forms.json``), exact
special cases, invariants that the definition implies, and a library routine
(PyTorch's CPU ``scaled_dot_product_attention`` in float64).  Together they are
chosen so that a plausible slip in the oracle -- a wrong sign, a dropped scale
or normalisation, swapped operands, a head or sequence index mix-up, an
off-by-one over the keys -- fails at least one of them (``test_oracle_mutants``
plants such slips and checks this).
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")
_SCALES = {"ln2": math.log(2.0), "ln3": math.log(3.0), "1": 1.0}


def _rand(lengths, h, d, seed, std=1.0):
    rng = np.random.default_rng(seed)
    t = int(sum(lengths))
    q = (rng.standard_normal((t, h, d)) * std).astype(np.float32)
    k = (rng.standard_normal((t, h, d)) * std).astype(np.float32)
    v = rng.standard_normal((t, h, d)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return q, k, v, cu


def _segments(cu):
    return [(int(cu[s]), int(cu[s + 1])) for s in range(len(cu) - 1)]


def pin_golden(lib):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], dtype=np.float32)
        k = np.array(c["k"], dtype=np.float32)
        v = np.array(c["v"], dtype=np.float32)
        exp = np.array([[[float(Fraction(x)) for x in hv] for hv in row] for row in c["expected"]])
        got = oracle.attention(q, k, v, c["cu_seqlens"], _SCALES[c["scale"]], lib=lib)
        assert np.allclose(got, exp, rtol=1e-13, atol=1e-13), (c["name"], got, exp)


def pin_scale_one_logistic(lib):
    # scale 1.0 (the Gemma 4V choice): logits (0, 1) give weights (1, e)/(1 + e)
    q = np.array([[[1.0]], [[0.0]]], np.float32)
    k = np.array([[[0.0]], [[1.0]]], np.float32)
    v = np.array([[[0.0]], [[1.0]]], np.float32)
    got = oracle.attention(q, k, v, [0, 2], 1.0, lib=lib)
    assert abs(got[0, 0, 0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(got[1, 0, 0] - 0.5) < 1e-15


def pin_single_key(lib):
    q, k, v, cu = _rand([1, 1, 1, 1], 3, 8, seed=11)
    got = oracle.attention(q, k, v, cu, 0.37, lib=lib)
    assert np.array_equal(got, v.astype(np.float64))


def pin_constant_v(lib):
    q, k, v, cu = _rand([5, 9, 2], 2, 6, seed=12, std=2.0)
    c = np.random.default_rng(13).standard_normal((1, 2, 6)).astype(np.float32)
    v = np.broadcast_to(c, v.shape).copy()
    got = oracle.attention(q, k, v, cu, 0.5, lib=lib)
    assert np.allclose(got, np.broadcast_to(c, got.shape), rtol=1e-14, atol=1e-14)


def pin_uniform_when_no_signal(lib):
    # Q = 0, or scale = 0: every key gets the same weight -> the sequence mean of V
    q, k, v, cu = _rand([4, 7, 3], 2, 5, seed=14)
    means = np.zeros(v.shape, np.float64)
    for a, b in _segments(cu):
        for h in range(v.shape[1]):
            for e in range(v.shape[2]):
                means[a:b, h, e] = math.fsum(float(x) for x in v[a:b, h, e]) / (b - a)
    got0 = oracle.attention(np.zeros_like(q), k, v, cu, 0.9, lib=lib)
    gots = oracle.attention(q, k, v, cu, 0.0, lib=lib)
    assert np.allclose(got0, means, rtol=1e-14, atol=1e-14)
    assert np.allclose(gots, means, rtol=1e-14, atol=1e-14)


def pin_weights_are_a_distribution(lib):
    # with V the identity over a sequence's keys, row i of the output is row i of the weights
    L = 6
    rng = np.random.default_rng(15)
    q = rng.standard_normal((L, 1, L)).astype(np.float32)
    k = rng.standard_normal((L, 1, L)).astype(np.float32)
    v = np.eye(L, dtype=np.float32)[:, None, :]
    got = oracle.attention(q, k, v, [0, L], 0.7, lib=lib)
    for i in range(L):
        p = oracle.row_probs(q, k, [0, L], 0.7, i, 0, lib=lib)
        assert abs(math.fsum(p) - 1.0) < 1e-14
        assert np.all(p > 0)
        assert np.allclose(got[i, 0, :], p, rtol=1e-14, atol=1e-15)
    # two keys: the weights are logistic in the logit difference
    p = oracle.row_probs(q[:2], k[:2], [0, 2], 0.7, 0, 0, lib=lib)
    d = 0.7 * (float(np.dot(q[0, 0].astype(np.float64), k[1, 0])) - float(np.dot(q[0, 0].astype(np.float64), k[0, 0])))
    assert abs(p[0] - 1.0 / (1.0 + math.exp(d))) < 1e-14


def pin_key_shift_invariance(lib):
    q, k, v, cu = _rand([6, 10], 2, 4, seed=16)
    k = (np.round(k * 64.0) / 64.0).astype(np.float32)  # coarse grid: k + u below is exact in float32
    base = oracle.attention(q, k, v, cu, 0.6, lib=lib)
    k2 = k.copy()
    u = np.array([[0.5, -0.25, 1.0, 0.125], [-1.0, 0.75, 0.0, 0.5]], np.float32)  # per head, exact in f32
    k2 += u[None]
    got = oracle.attention(q, k2, v, cu, 0.6, lib=lib)
    assert np.allclose(got, base, rtol=1e-12, atol=1e-12)


def pin_key_permutation_invariance(lib):
    q, k, v, cu = _rand([7, 5], 3, 4, seed=17)
    base = oracle.attention(q, k, v, cu, 0.8, lib=lib)
    perm = np.concatenate([np.random.default_rng(18).permutation(np.arange(a, b)) for a, b in _segments(cu)])
    # permute keys and values together; queries keep their rows
    got = oracle.attention(q, k[perm], v[perm], cu, 0.8, lib=lib)
    assert np.allclose(got, base, rtol=1e-13, atol=1e-13)


def pin_affine_in_v(lib):
    q, k, v, cu = _rand([8, 3], 2, 3, seed=19)
    v = (np.round(v * 64.0) / 64.0).astype(np.float32)  # coarse grid: 2v + 3 is exact in float32
    base = oracle.attention(q, k, v, cu, 0.5, lib=lib)
    got = oracle.attention(q, k, (2.0 * v + 3.0).astype(np.float32), cu, 0.5, lib=lib)
    assert np.allclose(got, 2.0 * base + 3.0, rtol=1e-13, atol=1e-13)


def pin_convex_hull(lib):
    q, k, v, cu = _rand([9, 4, 1], 2, 5, seed=20, std=3.0)
    got = oracle.attention(q, k, v, cu, 1.0, lib=lib)
    for a, b in _segments(cu):
        lo = v[a:b].min(axis=0).astype(np.float64)
        hi = v[a:b].max(axis=0).astype(np.float64)
        assert np.all(got[a:b] >= lo[None] - 1e-12) and np.all(got[a:b] <= hi[None] + 1e-12)


def pin_block_diagonal(lib):
    lengths = [5, 1, 8, 3]
    q, k, v, cu = _rand(lengths, 2, 4, seed=21)
    packed = oracle.attention(q, k, v, cu, 0.7, lib=lib)
    for a, b in _segments(cu):
        alone = oracle.attention(q[a:b], k[a:b], v[a:b], [0, b - a], 0.7, lib=lib)
        assert np.array_equal(alone, packed[a:b])
    # reordering the images reorders the output and changes nothing else
    order = [2, 0, 3, 1]
    segs = _segments(cu)
    idx = np.concatenate([np.arange(*segs[s]) for s in order])
    cu2 = np.concatenate([[0], np.cumsum([lengths[s] for s in order])]).astype(np.int32)
    re = oracle.attention(q[idx], k[idx], v[idx], cu2, 0.7, lib=lib)
    assert np.array_equal(re, packed[idx])


def pin_head_independence(lib):
    q, k, v, cu = _rand([6, 4], 3, 4, seed=22)
    base = oracle.attention(q, k, v, cu, 0.7, lib=lib)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, 1] += 1.0
    k2[:, 1] *= -2.0
    v2[:, 1] += 5.0
    got = oracle.attention(q2, k2, v2, cu, 0.7, lib=lib)
    assert np.array_equal(got[:, 0], base[:, 0]) and np.array_equal(got[:, 2], base[:, 2])
    assert not np.allclose(got[:, 1], base[:, 1])


def pin_head_dim_zero_padding(lib):
    q, k, v, cu = _rand([5, 6], 2, 3, seed=23)
    base = oracle.attention(q, k, v, cu, 0.45, lib=lib)
    pad = lambda x: np.concatenate([x, np.zeros(x.shape[:2] + (5,), np.float32)], axis=2)
    got = oracle.attention(pad(q), pad(k), pad(v), cu, 0.45, lib=lib)
    assert np.array_equal(got[:, :, :3], base) and np.all(got[:, :, 3:] == 0.0)


def pin_torch_sdpa(lib):
    # a library routine computing the same definition: PyTorch CPU SDPA in float64, per image
    import torch
    import torch.nn.functional as F
    lengths = [33, 1, 70, 17]
    q, k, v, cu = _rand(lengths, 4, 24, seed=24, std=1.5)
    got = oracle.attention(q, k, v, cu, 0.31, lib=lib)
    for a, b in _segments(cu):
        t = lambda x: torch.from_numpy(x[a:b].astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
        ref = F.scaled_dot_product_attention(t(q), t(k), t(v), scale=0.31)
        ref = ref.squeeze(0).permute(1, 0, 2).numpy()
        assert np.allclose(got[a:b], ref, rtol=1e-11, atol=1e-12)


def pin_rows_match_full(lib):
    q, k, v, cu = _rand([12, 5, 9], 2, 6, seed=25)
    full = oracle.attention(q, k, v, cu, 0.4, lib=lib)
    rows = np.array([0, 11, 12, 16, 17, 25, 3], np.int64)
    got = oracle.attention_rows(q, k, v, cu, 0.4, rows, lib=lib)
    assert np.array_equal(got, full[rows])


def _rand_gqa(lengths, h, hkv, d, seed, std=1.0):
    rng = np.random.default_rng(seed)
    t = int(sum(lengths))
    q = (rng.standard_normal((t, h, d)) * std).astype(np.float32)
    k = (rng.standard_normal((t, hkv, d)) * std).astype(np.float32)
    v = rng.standard_normal((t, hkv, d)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return q, k, v, cu


def pin_gqa_is_repeated_kv(lib):
    # grouped-query attention is multi-head attention on K/V whose head g is copied to the
    # H/Hkv consecutive query heads g*(H/Hkv) .. (g+1)*(H/Hkv)-1 ("hf2q ... vit_gpu.rs",
    # vit_repeat_kv_gpu doc); the copies are made here with numpy, outside the oracle
    for h, hkv in ((8, 2), (6, 3), (4, 1), (5, 5)):
        q, k, v, cu = _rand_gqa([9, 1, 23], h, hkv, 10, seed=26 + h + hkv, std=1.3)
        got = oracle.attention(q, k, v, cu, 0.37, lib=lib)
        ref = oracle.attention(q, np.repeat(k, h // hkv, axis=1), np.repeat(v, h // hkv, axis=1), cu, 0.37, lib=lib)
        assert np.array_equal(got, ref)
        rows = np.array([0, 8, 9, 10, 32], np.int64)
        assert np.array_equal(oracle.attention_rows(q, k, v, cu, 0.37, rows, lib=lib), ref[rows])


def pin_gqa_torch_sdpa(lib):
    # PyTorch's CPU SDPA in float64 with its own grouped-query mode
    import torch
    import torch.nn.functional as F
    q, k, v, cu = _rand_gqa([31, 4, 50], 8, 2, 16, seed=27, std=1.4)
    got = oracle.attention(q, k, v, cu, 0.29, lib=lib)
    for a, b in _segments(cu):
        t = lambda x: torch.from_numpy(x[a:b].astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
        ref = F.scaled_dot_product_attention(t(q), t(k), t(v), scale=0.29, enable_gqa=True)
        ref = ref.squeeze(0).permute(1, 0, 2).numpy()
        assert np.allclose(got[a:b], ref, rtol=1e-11, atol=1e-12)


def pin_gqa_constant_v_per_group(lib):
    # every key of K/V head g holding the value c_g makes every query head of group g output c_g
    q, k, v, cu = _rand_gqa([7, 19], 6, 3, 5, seed=28)
    for g in range(3):
        v[:, g, :] = np.float32(g + 0.25)
    got = oracle.attention(q, k, v, cu, 0.8, lib=lib)
    for h in range(6):
        assert np.allclose(got[:, h, :], h // 2 + 0.25, rtol=0, atol=1e-13)


# ---- masks: aligned causal ("hanzo-ml 0.11.4 src/vulkan_backend.rs", flash_attn_gpu doc)
# and a key window (the encoder attention meta of "inferencelayer 0.2.1 src/vision_gpu.rs",
# window 0 = unrestricted; read as |qi - kj| < window)

def pin_causal_torch_sdpa(lib):
    # PyTorch's CPU SDPA in float64 with its own causal flag (for as many queries as keys
    # it keeps key j <= query i), per image, also in its grouped-query mode
    import torch
    import torch.nn.functional as F
    for h, hkv, seed in ((4, 4, 40), (8, 2, 41)):
        q, k, v, cu = _rand_gqa([29, 1, 2, 64, 45], h, hkv, 12, seed=seed, std=1.4)
        got = oracle.attention(q, k, v, cu, 0.33, lib=lib, causal=True)
        for a, b in _segments(cu):
            t = lambda x: torch.from_numpy(x[a:b].astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
            ref = F.scaled_dot_product_attention(t(q), t(k), t(v), scale=0.33, is_causal=True,
                                                 enable_gqa=hkv != h)
            ref = ref.squeeze(0).permute(1, 0, 2).numpy()
            assert np.allclose(got[a:b], ref, rtol=1e-11, atol=1e-12)


def pin_causal_first_row_is_its_value(lib):
    # the first token of an image sees only itself: its output is its own value row, exactly
    q, k, v, cu = _rand([5, 1, 17], 3, 8, seed=42, std=2.0)
    got = oracle.attention(q, k, v, cu, 0.9, lib=lib, causal=True)
    for a, _ in _segments(cu):
        assert np.array_equal(got[a], v[a].astype(np.float64))


def pin_window_one_is_identity(lib):
    # window 1 keeps only the key at the query's own position: O = V exactly, with or without causal
    q, k, v, cu = _rand([9, 1, 33], 2, 8, seed=43, std=3.0)
    for causal in (False, True):
        got = oracle.attention(q, k, v, cu, 0.7, lib=lib, causal=causal, window=1)
        assert np.array_equal(got, v.astype(np.float64))


def _slice_attention(lib, q, k, v, i, lo, hi, scale):
    """Unmasked attention of query row i over the keys [lo, hi) only, through the mask-free
    oracle: one image of hi - lo rows whose queries are copies of row i and whose keys and
    values are rows lo .. hi-1 (cut out with numpy)."""
    n = hi - lo
    qx = np.repeat(q[i:i + 1], n, axis=0)
    return oracle.attention(qx, k[lo:hi], v[lo:hi], [0, n], scale, lib=lib)[0]


def pin_causal_is_prefix_attention(lib):
    # causal row i is bidirectional attention over the image's prefix [a, i]
    q, k, v, cu = _rand([23, 40], 2, 10, seed=44, std=1.6)
    got = oracle.attention(q, k, v, cu, 0.45, lib=lib, causal=True)
    for a, b in _segments(cu):
        for i in (a, a + 1, a + 7, b - 2, b - 1):
            ref = _slice_attention(lib, q, k, v, i, a, i + 1, 0.45)
            assert np.allclose(got[i], ref, rtol=1e-13, atol=1e-14)


def pin_window_is_band_attention(lib):
    # window W: row i is bidirectional attention over the keys [i-W+1, i+W) clipped to its
    # image, and with causal over [i-W+1, i]
    q, k, v, cu = _rand([37, 6, 50], 2, 8, seed=45, std=1.5)
    for w in (2, 5, 16):
        for causal in (False, True):
            got = oracle.attention(q, k, v, cu, 0.5, lib=lib, causal=causal, window=w)
            for a, b in _segments(cu):
                for i in sorted({a, a + 1, a + 3, (a + b) // 2, b - 3, b - 1} & set(range(a, b))):
                    lo, hi = max(a, i - w + 1), (i + 1 if causal else min(b, i + w))
                    ref = _slice_attention(lib, q, k, v, i, lo, hi, 0.5)
                    assert np.allclose(got[i], ref, rtol=1e-13, atol=1e-14), (w, causal, i)


def pin_wide_window_is_no_window(lib):
    # a window at least as long as every image changes nothing (the same sums, bit for bit)
    q, k, v, cu = _rand([12, 30, 1], 2, 6, seed=46)
    for causal in (False, True):
        ref = oracle.attention(q, k, v, cu, 0.6, lib=lib, causal=causal)
        for w in (30, 31, 1000):
            assert np.array_equal(oracle.attention(q, k, v, cu, 0.6, lib=lib, causal=causal, window=w), ref)


def pin_masked_rows_match_full(lib):
    q, k, v, cu = _rand_gqa([12, 5, 30], 4, 2, 6, seed=47)
    rows = np.array([0, 11, 12, 16, 17, 25, 46, 3], np.int64)
    for causal, w in ((True, 0), (False, 4), (True, 7)):
        full = oracle.attention(q, k, v, cu, 0.4, lib=lib, causal=causal, window=w)
        got = oracle.attention_rows(q, k, v, cu, 0.4, rows, lib=lib, causal=causal, window=w)
        assert np.array_equal(got, full[rows])


# ---- the input side: qkv split, per-head RMS norm, rope ("inferencelayer 0.2.1
# src/vision_gpu.rs", VIS_QKV_ROPE and GLM_QKV_QKNORM_ROPE; "hf2q ... vit_gpu.rs",
# vit_rms_norm_gpu: eps inside the square root)

def _packed(t, h, g, d, seed, std=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((t, (h + 2 * g) * d)) * std).astype(np.float32), rng


def pin_prologue_split_is_exact(lib):
    # no tables and no gains: Q, K and V are the packed row's head slots, bit for bit
    for h, g in ((4, 4), (6, 2), (3, 1)):
        x, _ = _packed(5, h, g, 8, seed=60 + h)
        q, k, v = oracle.qkv_prologue(x, h, g, lib=lib)
        assert np.array_equal(q, x[:, :h * 8].reshape(5, h, 8).astype(np.float64))
        assert np.array_equal(k, x[:, h * 8:(h + g) * 8].reshape(5, g, 8).astype(np.float64))
        assert np.array_equal(v, x[:, (h + g) * 8:].reshape(5, g, 8).astype(np.float64))


def pin_prologue_rope_quarter_turn(lib):
    # cos = 1, sin = 0 is the identity; cos = 0, sin = 1 is rotate_half itself: the low half
    # takes minus the high half, the high half takes the low half (values exact)
    x, _ = _packed(3, 2, 1, 8, seed=62)
    one, zero = np.ones((3, 8), np.float32), np.zeros((3, 8), np.float32)
    q, k, v = oracle.qkv_prologue(x, 2, 1, cos=one, sin=zero, lib=lib)
    assert np.array_equal(q, x[:, :16].reshape(3, 2, 8).astype(np.float64))
    q, k, v = oracle.qkv_prologue(x, 2, 1, cos=zero, sin=one, lib=lib)
    xq = x[:, :16].reshape(3, 2, 8).astype(np.float64)
    assert np.array_equal(q[..., :4], -xq[..., 4:]) and np.array_equal(q[..., 4:], xq[..., :4])
    xk = x[:, 16:24].reshape(3, 1, 8).astype(np.float64)
    assert np.array_equal(k[..., :4], -xk[..., 4:]) and np.array_equal(k[..., 4:], xk[..., :4])
    assert np.array_equal(v, x[:, 24:].reshape(3, 1, 8).astype(np.float64))  # V is never rotated


def _angle_tables(t, d, seed):
    # standard rope tables: the angle of dim j equals that of dim j + d/2
    rng = np.random.default_rng(seed)
    ang = rng.uniform(-4, 4, size=(t, d // 2))
    ang = np.concatenate([ang, ang], axis=1)
    return ang, np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def pin_prologue_rope_is_a_rotation(lib):
    # with tables of one angle per pair (j, j + d/2) the rope rotates each pair: norms are
    # kept, and dot products of two rotated rows depend only on the angle difference
    t, h, d = 6, 2, 16
    x, _ = _packed(t, h, h, d, seed=63)
    ang, c, s_ = _angle_tables(t, d, 64)
    q, k, _ = oracle.qkv_prologue(x, h, h, cos=c, sin=s_, lib=lib)
    q0 = x[:, :h * d].reshape(t, h, d).astype(np.float64)
    assert np.allclose(np.linalg.norm(q, axis=-1), np.linalg.norm(q0, axis=-1), rtol=1e-6, atol=0)
    # rotating rows i and j by their angles gives the same dot product as rotating row i by
    # the difference alone (tables recomputed in float64 and rounded like the others)
    i, j = 1, 4
    diff = ang[i] - ang[j]
    c2, s2 = np.cos(diff).astype(np.float32)[None], np.sin(diff).astype(np.float32)[None]
    qi, _, _ = oracle.qkv_prologue(x[i:i + 1], h, h, cos=c2, sin=s2, lib=lib)
    kj = x[j:j + 1, h * d:2 * h * d].reshape(1, h, d).astype(np.float64)
    lhs = np.sum(q[i] * k[j], axis=-1)
    rhs = np.sum(qi[0] * kj[0], axis=-1)
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-5)


def pin_prologue_rms_norm_closed_form(lib):
    # a constant head vector c: mean of squares c^2, so y = c / sqrt(c^2 + eps) * gain
    t, h, d, eps = 2, 2, 8, 0.5
    x = np.full((t, 3 * h * d), 1.5, np.float32)  # H = Hkv = h: width (h + 2h) d
    w = np.arange(1, d + 1, dtype=np.float32)
    q, k, v = oracle.qkv_prologue(x, h, h, q_weight=w, k_weight=2 * w, eps=eps, lib=lib)
    assert np.allclose(q, 1.5 / np.sqrt(2.25 + eps) * w, rtol=1e-14, atol=0)
    assert np.allclose(k, 1.5 / np.sqrt(2.25 + eps) * 2 * w, rtol=1e-14, atol=0)
    assert np.array_equal(v, np.full_like(v, 1.5))


def pin_prologue_rms_norm_torch(lib):
    # PyTorch's rms_norm (float64) per head, with a gain and eps = 0.1
    import torch
    import torch.nn.functional as F
    t, h, g, d = 7, 4, 2, 16
    x, rng = _packed(t, h, g, d, seed=65, std=2.0)
    qw = rng.uniform(0.5, 1.5, d).astype(np.float32)
    kw = rng.uniform(0.5, 1.5, d).astype(np.float32)
    q, k, _ = oracle.qkv_prologue(x, h, g, q_weight=qw, k_weight=kw, eps=0.1, lib=lib)
    xt = torch.from_numpy(x.astype(np.float64))
    rq = F.rms_norm(xt[:, :h * d].reshape(t, h, d), (d,), torch.from_numpy(qw.astype(np.float64)), 0.1)
    rk = F.rms_norm(xt[:, h * d:(h + g) * d].reshape(t, g, d), (d,), torch.from_numpy(kw.astype(np.float64)), 0.1)
    assert np.allclose(q, rq.numpy(), rtol=1e-12, atol=1e-13)
    assert np.allclose(k, rk.numpy(), rtol=1e-12, atol=1e-13)


def pin_prologue_norm_then_rope(lib):
    # the norm comes first: norm + rope equals the rope applied (as a second call, with no
    # gains) to the normed rows; with a non-uniform gain the other order differs
    t, h, d = 4, 2, 16
    x, rng = _packed(t, h, h, d, seed=66)
    _, c, s_ = _angle_tables(t, d, 67)
    w = rng.uniform(0.2, 2.0, d).astype(np.float32)
    q, k, _ = oracle.qkv_prologue(x, h, h, cos=c, sin=s_, q_weight=w, k_weight=w, eps=1e-3, lib=lib)
    qn, kn, vn = oracle.qkv_prologue(x, h, h, q_weight=w, k_weight=w, eps=1e-3, lib=lib)
    packed = np.concatenate([qn.reshape(t, -1), kn.reshape(t, -1), vn.reshape(t, -1)], axis=1)
    q2, k2, _ = oracle.qkv_prologue(packed.astype(np.float32), h, h, cos=c, sin=s_, lib=lib)
    assert np.allclose(q, q2, rtol=1e-6, atol=1e-6) and np.allclose(k, k2, rtol=1e-6, atol=1e-6)


PINS = [
    pin_golden, pin_scale_one_logistic, pin_single_key, pin_constant_v, pin_uniform_when_no_signal,
    pin_weights_are_a_distribution, pin_key_shift_invariance, pin_key_permutation_invariance,
    pin_affine_in_v, pin_convex_hull, pin_block_diagonal, pin_head_independence,
    pin_head_dim_zero_padding, pin_torch_sdpa, pin_rows_match_full,
    pin_gqa_is_repeated_kv, pin_gqa_torch_sdpa, pin_gqa_constant_v_per_group,
    pin_causal_torch_sdpa, pin_causal_first_row_is_its_value, pin_window_one_is_identity,
    pin_causal_is_prefix_attention, pin_window_is_band_attention, pin_wide_window_is_no_window,
    pin_masked_rows_match_full,
    pin_prologue_split_is_exact, pin_prologue_rope_quarter_turn, pin_prologue_rope_is_a_rotation,
    pin_prologue_rms_norm_closed_form, pin_prologue_rms_norm_torch, pin_prologue_norm_then_rope,
]
