"""The qkv prologue on the HIP path vs the float64 oracle, through the C ABI.

Tolerances by output kind: a 16-bit output is the oracle's value rounded to that kind, up to
one unit in its last place (float32 arithmetic may land on the other side of a rounding
midpoint): 2^-7 |ref| for bfloat16 (8 significant bits), 2^-10 |ref| for half (11), plus half's
smallest subnormal; float32 outputs 2^-20 |ref|.  On top, 2^-20 of the element's rope pair
norm sqrt(ref[d]^2 + ref[d +- D/2]^2): the rope adds two products that may cancel, each as
large as the pair (a rotation keeps the pair's norm), and the float32 rounding of the norm and
the products is relative to them, not to the sum.  The split alone and the rope at a quarter
turn move or negate values and must be exact.
"""
import numpy as np
import pytest
import torch

import oracle
import vision_transformer_attention_amd as vta
from gpu_util import DEV, TOL, max_abs_err, say
from vision_transformer_attention_amd import inputs

pytestmark = pytest.mark.gpu

REL = {inputs.BF16: 2.0 ** -7, inputs.F16: 2.0 ** -10, inputs.F32: 2.0 ** -20}
ABS = {inputs.BF16: 1e-30, inputs.F16: 2.0 ** -24, inputs.F32: 1e-30}


def _gpu(d, out=None):
    dev = torch.device(DEV)
    mv = lambda x: x.to(dev) if x is not None else None
    res = vta.qkv_prologue(mv(d["qkv"]), d["n_heads"], d["n_kv_heads"], mv(d["cos"]), mv(d["sin"]),
                           mv(d["q_weight"]), mv(d["k_weight"]), eps=1e-6, out=out)
    torch.cuda.synchronize()
    return [x.cpu() for x in res]


def _check(d, dtype, label):
    got = _gpu(d)
    ref = oracle.qkv_prologue(d["qkv"], d["n_heads"], d["n_kv_heads"], d["cos"], d["sin"], d["q_weight"],
                              d["k_weight"], eps=1e-6)
    for name, g, r in zip("qkv", got, ref):
        gv = g.float().numpy().astype(np.float64)
        pair = np.sqrt(r * r + np.roll(r, r.shape[-1] // 2, axis=-1) ** 2)
        bound = REL[dtype] * np.abs(r) + 2.0 ** -20 * pair + ABS[dtype]
        excess = np.abs(gv - r) - bound
        worst = float(excess.max()) if excess.size else -1.0
        say(f"[prologue] {label} {name}: max |err| {float(np.abs(gv - r).max()) if r.size else 0:.3e}, "
            f"worst margin {worst:.3e}")
        assert worst <= 0.0, (label, name)
    return got


@pytest.mark.parametrize("rope,norm", [(True, True), (True, False), (False, True)])
@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.F16, inputs.F32])
@pytest.mark.parametrize("head_dim", [64, 72, 80, 128])
def test_prologue_matches_oracle(head_dim, dtype, rope, norm):
    d = inputs.prologue_inputs([1, 7, 300, 33], n_heads=4, head_dim=head_dim, dtype=dtype, seed=70 + head_dim,
                               n_kv_heads=2, rope=rope, norm=norm)
    _check(d, dtype, f"D={head_dim} {dtype} rope={rope} norm={norm}")


@pytest.mark.parametrize("h,hkv", [(16, 16), (16, 4), (8, 1), (3, 3)])
def test_prologue_head_layouts(h, hkv):
    d = inputs.prologue_inputs([129, 1, 64], n_heads=h, head_dim=80, dtype=inputs.BF16, seed=71 + h + hkv,
                               n_kv_heads=hkv)
    _check(d, inputs.BF16, f"H={h} Hkv={hkv}")


@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.F16, inputs.F32])
def test_prologue_split_and_quarter_turn_are_exact(dtype):
    d = inputs.prologue_inputs([50, 13], n_heads=6, head_dim=72, dtype=dtype, seed=72, n_kv_heads=3, rope=False,
                               norm=False)
    q, k, v = _gpu(d)
    x = d["qkv"]
    t, dd = x.shape[0], 72
    assert torch.equal(q, x[:, :6 * dd].reshape(t, 6, dd))
    assert torch.equal(k, x[:, 6 * dd:9 * dd].reshape(t, 3, dd))
    assert torch.equal(v, x[:, 9 * dd:].reshape(t, 3, dd))
    d["cos"], d["sin"] = torch.zeros(t, dd), torch.ones(t, dd)  # rope by a quarter turn: rotate_half exactly
    q, k, v = _gpu(d)
    xq = x[:, :6 * dd].reshape(t, 6, dd)
    assert torch.equal(q[..., :36], -xq[..., 36:]) and torch.equal(q[..., 36:], xq[..., :36])
    assert torch.equal(v, x[:, 9 * dd:].reshape(t, 3, dd))


def test_prologue_full_packed_batch_and_out_buffers():
    # the packed batch's shape (17,408 tokens, 16 heads of 80, bf16), written into given buffers
    d = inputs.prologue_inputs(inputs.PACKED_LENGTHS, n_heads=16, head_dim=80, dtype=inputs.BF16, seed=73)
    dev = torch.device(DEV)
    t = d["qkv"].shape[0]
    out = tuple(torch.full((t, 16, 80), float("nan"), dtype=torch.bfloat16, device=dev) for _ in range(3))
    got = _gpu(d, out=out)
    ref = oracle.qkv_prologue(d["qkv"], 16, 16, d["cos"], d["sin"], d["q_weight"], d["k_weight"], eps=1e-6)
    for g, r in zip(got, ref):
        pair = np.sqrt(r * r + np.roll(r, 40, axis=-1) ** 2)
        excess = np.abs(g.float().numpy().astype(np.float64) - r) - REL[inputs.BF16] * np.abs(r) - 2.0 ** -20 * pair
        assert float(excess.max()) <= 0.0


@pytest.mark.parametrize("dtype,head_dim", [(inputs.BF16, 80), (inputs.F16, 72), (inputs.F32, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_prologue_then_attention(causal, dtype, head_dim):
    # the whole path: the prologue and the attention on the GPU against the oracle's prologue
    # (its outputs rounded to the element kind, as the GPU's are) and the oracle's attention
    lengths = [257, 64, 1, 130]
    d = inputs.prologue_inputs(lengths, n_heads=8, head_dim=head_dim, dtype=dtype, seed=74, n_kv_heads=2)
    dev = torch.device(DEV)
    mv = lambda x: x.to(dev) if x is not None else None
    q, k, v = vta.qkv_prologue(mv(d["qkv"]), 8, 2, mv(d["cos"]), mv(d["sin"]), mv(d["q_weight"]),
                               mv(d["k_weight"]), eps=1e-6)
    cu = d["cu_seqlens"]
    scale = head_dim ** -0.5
    o = vta.fwd(q, k, v, cu.to(dev), scale, causal=causal).cpu()
    rq, rk, rv = oracle.qkv_prologue(d["qkv"], 8, 2, d["cos"], d["sin"], d["q_weight"], d["k_weight"], eps=1e-6)
    kind = {inputs.BF16: torch.bfloat16, inputs.F16: torch.float16, inputs.F32: torch.float32}[dtype]
    b = lambda a: torch.from_numpy(a).to(kind)
    ref = oracle.attention(b(rq), b(rk), b(rv), cu, scale, causal=causal)
    err, where = max_abs_err(o, ref)
    say(f"[prologue] prologue + attention {dtype} D={head_dim} causal={causal}: max-abs err {err:.3e} at {where}")
    assert err <= TOL[dtype]
