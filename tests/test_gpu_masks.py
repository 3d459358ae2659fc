"""Masked attention (aligned causal and a key window) on the HIP path vs the float64 oracle.

Causal: inside each image, query qi sees keys kj <= qi ("hanzo-ml 0.11.4
src/vulkan_backend.rs", flash_attn_gpu doc, aligned causal with as many keys as queries).
Window w > 0: keys with |qi - kj| < w (the encoder attention meta's window of
"inferencelayer 0.2.1 src/vision_gpu.rs", 0 = unrestricted, read as this band).  The
tolerances are those of the unmasked path (``gpu_util.TOL``).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import vision_transformer_attention_amd as vta
from gpu_util import DEV, TOL, check_workload, max_abs_err, run_gpu, sample_rows, say
from vision_transformer_attention_amd import binding, inputs

pytestmark = pytest.mark.gpu

EDGE = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300]
# narrow windows (a query sees < 1024 keys) run the masked kernel with small query blocks, the
# causal mask and wide windows the one with large blocks
MASKS = [(True, 0), (False, 1), (False, 2), (False, 33), (False, 100), (True, 16), (True, 64), (True, 129),
         (False, 200), (False, 513), (True, 1024)]


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("head_dim", [64, 72, 80, 128])
def test_masked_edge_lengths_bf16(head_dim, causal, window):
    w = inputs.custom(EDGE, n_heads=2, head_dim=head_dim, dtype=inputs.BF16, seed=300 + head_dim)
    check_workload(w, full=True, causal=causal, window=window)


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 31), (True, 65)])
@pytest.mark.parametrize("dtype,head_dim", [(inputs.F32, 64), (inputs.F32, 80), (inputs.F32, 128),
                                             (inputs.F16, 72), (inputs.F16, 128)])
def test_masked_edge_lengths_f32_and_half(dtype, head_dim, causal, window):
    w = inputs.custom(EDGE, n_heads=2, head_dim=head_dim, dtype=dtype, seed=320 + head_dim)
    check_workload(w, full=True, causal=causal, window=window)


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 40), (True, 300), (False, 600), (True, 1100)])
@pytest.mark.parametrize("dtype,head_dim", [(inputs.BF16, 80), (inputs.BF16, 128), (inputs.F16, 64),
                                             (inputs.F32, 80)])
def test_masked_rising_and_jumping_scores(dtype, head_dim, causal, window):
    # scores drift by hundreds of log2 units along each image and jump at spike keys: rows
    # first see a key in different steps and raise their offsets many times under the mask.
    # Float32 inputs drift by 40 (scores up to ~250): at 300 the scores reach ~1850, where
    # one float32 rounding of a score is ~1e-4 and a plain float32 evaluation of the same
    # attention on the CPU already misses the 1e-4 bound.
    ramp = 40.0 if dtype == inputs.F32 else 300.0
    w = inputs.custom([1000, 777, 64, 33, 5], n_heads=2, head_dim=head_dim, dtype=dtype, seed=29, key_ramp=ramp,
                      spikes=2)
    check_workload(w, full=True, causal=causal, window=window)


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 24), (True, 50)])
def test_masked_grouped_query(causal, window):
    w = inputs.custom([129, 1, 64, 200, 33], n_heads=8, head_dim=80, dtype=inputs.BF16, seed=31, n_kv_heads=2)
    check_workload(w, full=True, causal=causal, window=window)


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 256), (True, 256), (False, 700), (True, 2000)])
def test_masked_packed_varlen_sampled_rows(causal, window):
    # the benchmark's packed batch at full size, in the launch the benchmark makes
    check_workload(inputs.WORKLOADS["packed-varlen-8"], full=False, causal=causal, window=window)


def test_causal_page_912_full():
    check_workload(inputs.WORKLOADS["page-912"], full=True, causal=True)


def test_causal_many_images_and_one_long_image():
    # more images than the launch sorts (the causal items then keep the image order), and one
    # image with more query blocks than the cost-ordered plan lists (it keeps the image plan)
    rng = np.random.default_rng(38)
    lengths = [int(x) for x in rng.integers(1, 90, size=300)]
    w = inputs.custom(lengths, n_heads=2, head_dim=64, dtype=inputs.BF16, seed=38)
    check_workload(w, full=True, causal=True)
    w = inputs.custom([40000], n_heads=1, head_dim=80, dtype=inputs.BF16, seed=39)
    rows = np.array([0, 1, 63, 64, 20000, 32767, 32768, 39998, 39999], np.int64)
    check_workload(w, full=False, rows=rows, causal=True)
    check_workload(w, full=False, rows=rows, causal=True, window=3000)


@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.F16, inputs.F32])
def test_window_one_returns_v_exactly(dtype):
    # each query sees only its own key.  In the 16-bit kernels its one weight, rounded, is a
    # power of two that the row sum divides out exactly: o is v bit for bit.  In float32 the
    # weight is exp2 of a rounding residue, and o = (w*v)*(1/w) is v within a few ulps.
    w = inputs.custom([1, 17, 300, 64], n_heads=3, head_dim=80, dtype=dtype, seed=33)
    q, k, v, cu, scale = inputs.make(w)
    for causal in (False, True):
        o = run_gpu(q, k, v, cu, scale, causal=causal, window=1)
        if dtype == inputs.F32:
            assert torch.allclose(o, v, rtol=1e-6, atol=0.0), causal
        else:
            assert torch.equal(o, v), causal


@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.F32])
def test_no_mask_through_masked_entry_is_bitwise_unmasked(dtype):
    w = inputs.custom([300, 5, 129], n_heads=4, head_dim=64, dtype=dtype, seed=34, n_kv_heads=2)
    q, k, v, cu, scale = inputs.make(w)
    ref = run_gpu(q, k, v, cu, scale)
    d = torch.device(DEV)
    qd, kd, vd, cud = q.to(d), k.to(d), v.to(d), cu.to(d)
    o = torch.empty_like(qd)
    code = binding._call_code(qd.dtype, qd.dtype)
    binding.fwd_masked_raw(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), cud.data_ptr(), 3, 4, 2, 64,
                           scale, 0, 0, code, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), ref)


def test_wide_window_matches_no_window():
    w = inputs.custom([300, 5, 129], n_heads=2, head_dim=80, dtype=inputs.BF16, seed=35)
    q, k, v, cu, scale = inputs.make(w)
    ref = oracle.attention(q, k, v, cu, scale)
    for causal, win in ((False, 300), (False, 10 ** 6), (True, 10 ** 6)):
        o = run_gpu(q, k, v, cu, scale, causal=causal, window=win)
        r = ref if not causal else oracle.attention(q, k, v, cu, scale, causal=True)
        err, where = max_abs_err(o, r)
        say(f"[masks] window {win} causal {causal}: err {err:.3e} at {where}")
        assert err <= TOL[inputs.BF16]


@pytest.mark.parametrize("scale", [0.0, -0.4, 1.0])
def test_masked_scale_is_passed_through(scale):
    w = inputs.custom([97, 1, 200], n_heads=2, head_dim=64, dtype=inputs.BF16, seed=36)
    q, k, v, cu, _ = inputs.make(w)
    for causal, win in ((True, 0), (False, 20)):
        o = run_gpu(q, k, v, cu, scale, causal=causal, window=win)
        err, where = max_abs_err(o, oracle.attention(q, k, v, cu, scale, causal=causal, window=win))
        say(f"[masks] scale {scale} causal {causal} window {win}: err {err:.3e} at {where}")
        assert err <= TOL[inputs.BF16]


@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.F16])
def test_masked_float32_output(dtype):
    w = inputs.custom(EDGE, n_heads=2, head_dim=80, dtype=dtype, seed=37)
    o, _ = check_workload(w, full=True, out_dtype=torch.float32, causal=True, window=70)
    q, k, v, cu, scale = inputs.make(w)
    o16 = run_gpu(q, k, v, cu, scale, causal=True, window=70)
    assert torch.equal(o.to(o16.dtype), o16)  # the 16-bit output is the float32 one rounded


def test_masked_deterministic_bitwise():
    w = inputs.WORKLOADS["packed-varlen-8"]
    q, k, v, cu, scale = inputs.make(w)
    a = run_gpu(q, k, v, cu, scale, causal=True, window=200)
    b = run_gpu(q, k, v, cu, scale, causal=True, window=200)
    assert torch.equal(a, b)
