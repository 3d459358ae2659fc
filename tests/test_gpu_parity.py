"""HIP path vs the float64 oracle, element by element, through the C ABI.

Tolerances: max-abs 1e-4 for float32 inputs, 2e-2 for bfloat16 and 1e-2 for half inputs
(``gpu_util.TOL`` derives the last).
The small workloads are compared in full; the packed batch and the long
sequence (full size, same launch as the benchmark) on sampled rows that cover
every image's first and last rows and tile boundaries, plus properties that hold
at any size.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, check_workload, run_gpu, say, sample_rows
from vision_transformer_attention_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny-64", "vit-196", "page-912"])
def test_workload_full(name):
    check_workload(inputs.WORKLOADS[name], full=True)


def test_packed_varlen_every_row():
    # the full packed batch, every one of its 17,408 rows (the launch the benchmark times)
    check_workload(inputs.WORKLOADS["packed-varlen-8"], full=True)


def long_rows() -> np.ndarray:
    """1,024 rows of the 16,384-token sequence: at head_dim 128 a work item is 128 query rows,
    4 wavefronts of two 16-row blocks; every item contributes one row of every block of every
    wavefront, at a lane position that varies from item to item, plus the sequence's ends."""
    rows = []
    for item in range(128):
        for wave in range(4):
            for qb in range(2):
                rows.append(item * 128 + wave * 32 + qb * 16 + (item * 7 + wave * 3 + qb * 5) % 16)
    rows = sorted(set(rows) | {0, 1, 16382, 16383})
    return np.array(rows, np.int64)


def test_long_sequence_rows_of_every_item_and_convex_hull():
    w = inputs.WORKLOADS["long-16384"]
    rows = long_rows()
    assert len(rows) >= 1024
    o, _ = check_workload(w, full=False, rows=rows)
    _, _, v, _, _ = inputs.make(w)
    vf, of = v.float(), o.float()
    lo, hi = vf.min(dim=0).values, vf.max(dim=0).values
    assert bool((of >= lo - 2e-2).all()) and bool((of <= hi + 2e-2).all())


@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.F32])
@pytest.mark.parametrize("head_dim", [64, 72, 80, 128])
def test_edge_lengths(dtype, head_dim):
    lengths = [1, 2, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 255, 300]
    w = inputs.custom(lengths, n_heads=3, head_dim=head_dim, dtype=dtype, seed=100 + head_dim)
    check_workload(w, full=True)


@pytest.mark.parametrize("dtype,head_dim", [(inputs.BF16, 64), (inputs.BF16, 80), (inputs.BF16, 128),
                                             (inputs.F32, 80)])
def test_rising_and_jumping_scores(dtype, head_dim):
    # Scores drift by hundreds of log2 units along each sequence (up for some queries, down
    # for others) and jump at a few spike keys, so the running max is raised many times,
    # sometimes by far more than the exponent range.  Float32 inputs drift by 40 (scores up
    # to ~250): at 300 the scores reach ~1850, where one float32 rounding of a score is ~1e-4
    # and a plain float32 evaluation on the CPU already misses the 1e-4 bound.
    ramp = 40.0 if dtype == inputs.F32 else 300.0
    w = inputs.custom([1000, 777, 64, 33, 5], n_heads=2, head_dim=head_dim, dtype=dtype, seed=23, key_ramp=ramp,
                      spikes=2)
    check_workload(w, full=True)


@pytest.mark.parametrize("head_dim", [64, 80])
def test_rising_and_jumping_scores_in_large_items(head_dim):
    # The same drift and spikes at 16 heads over long images, so that the launch runs its
    # 256-query items (the path of the packed batch) and raises their offsets many times.
    w = inputs.custom([3000, 2500, 1200, 777, 33, 5], n_heads=16, head_dim=head_dim, dtype=inputs.BF16, seed=29,
                      key_ramp=300.0, spikes=2)
    check_workload(w, full=True)


@pytest.mark.parametrize("scale", [1.0, 0.0, -0.3, 2.5])
def test_scale_is_passed_through(scale):
    w = inputs.custom([77, 200], n_heads=2, head_dim=64, dtype=inputs.BF16, seed=9, std=0.7, scale=scale)
    check_workload(w, full=True)


def test_zero_length_sequences_between():
    w = inputs.custom([0, 40, 0, 0, 129, 1, 0], n_heads=2, head_dim=80, dtype=inputs.BF16, seed=11)
    check_workload(w, full=True)


def test_many_sequences_unsorted_and_split_launches():
    rng = np.random.default_rng(12)
    lengths = rng.integers(0, 40, size=700).tolist()  # > 512 sequences: several launches
    w = inputs.custom(lengths, n_heads=2, head_dim=72, dtype=inputs.BF16, seed=12)
    check_workload(w, full=True)


@pytest.mark.parametrize("head_dim", [80, 128])
def test_one_image_at_an_offset_through_the_raw_abi(head_dim):
    # A launch over one image takes a closed-form plan; its rows [a, b) need not start at row
    # 0 of the buffers (cu_seqlens[0] is the image's first row).  Rows outside the image, and
    # every row of a launch over one empty image, keep what the output held.
    from vision_transformer_attention_amd import binding
    t, a, b = 300, 37, 237
    w = inputs.custom([t], n_heads=3, head_dim=head_dim, dtype=inputs.BF16, seed=15)
    q, k, v, _cu, scale = inputs.make(w)
    d = torch.device("cuda:0")
    qd, kd, vd = q.to(d), k.to(d), v.to(d)
    sentinel = torch.full_like(qd, 7.0)
    for lo, hi in ((a, b), (100, 100), (a, a + 1)):
        say(f"one image rows [{lo}, {hi}) of {t}, head_dim {head_dim}")
        o = sentinel.clone()
        cu = torch.tensor([lo, hi], dtype=torch.int32, device=d)
        binding.fwd_raw(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), cu.data_ptr(), 1, 3, head_dim,
                        scale, binding.DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        o = o.cpu()
        assert torch.equal(o[:lo], sentinel[:lo].cpu()) and torch.equal(o[hi:], sentinel[hi:].cpu())
        if hi > lo:
            alone = run_gpu(q[lo:hi].contiguous(), k[lo:hi].contiguous(), v[lo:hi].contiguous(),
                            torch.tensor([0, hi - lo], dtype=torch.int32), scale)
            assert torch.equal(o[lo:hi], alone)  # the same launch on its own buffers
            ref = oracle.attention(q[lo:hi], k[lo:hi], v[lo:hi], torch.tensor([0, hi - lo], dtype=torch.int32),
                                   scale)
            err = float(np.max(np.abs(o[lo:hi].float().numpy().astype(np.float64) - ref)))
            assert err <= TOL[inputs.BF16], err


def test_default_call_does_not_synchronise():
    # With cu_seqlens on the device the default call only enqueues work: under torch's
    # sync debug mode "error" any host synchronisation (such as reading cu_seqlens back
    # for a check) raises.
    import vision_transformer_attention_amd as vta
    w = inputs.custom([300, 129, 1, 64], n_heads=4, head_dim=80, dtype=inputs.BF16, seed=31)
    q, k, v, cu, scale = inputs.make(w)
    d = torch.device("cuda:0")
    qd, kd, vd, cud = q.to(d), k.to(d), v.to(d), cu.to(d)
    vta.fwd(qd, kd, vd, cud, scale)  # device set-up (kernel table) outside the checked region
    torch.cuda.synchronize()
    torch.cuda.set_sync_debug_mode("error")
    try:
        o = vta.fwd(qd, kd, vd, cud, scale)
        oc = vta.fwd(qd, kd, vd, cud, scale, causal=True, out_dtype=torch.float32)
    finally:
        torch.cuda.set_sync_debug_mode("default")
    torch.cuda.synchronize()
    for got, causal in ((o, False), (oc, True)):
        ref = oracle.attention(q, k, v, cu, scale, causal=causal)
        err = float(np.max(np.abs(got.float().cpu().numpy().astype(np.float64) - ref)))
        say(f"[parity] async default call causal={causal}: max-abs err {err:.3e}")
        assert err <= TOL[inputs.BF16], err


@pytest.mark.parametrize("length,causal", [(1024, False), (1025, False), (3840, False), (3841, False),
                                           (3841, True), (64, True)])
def test_one_image_on_both_sides_of_the_item_size_thresholds(length, causal):
    # A launch over one image chooses its item size in closed form: at 16 heads and a 512-
    # workgroup grid, up to 1024 tokens take key-split 32-query items, up to 3840 64-query
    # items, and longer images 256-query items (a masked launch never splits by keys).
    w = inputs.custom([length], n_heads=16, head_dim=64, dtype=inputs.BF16, seed=17 + length)
    check_workload(w, full=False, causal=causal)


@pytest.mark.parametrize("causal", [False, True])
def test_hip_graph_capture_and_replay(causal):
    # With out= given and the host-side cu_seqlens check off, a call allocates nothing and never
    # waits on the device, so it can be captured into a HIP graph.  Each replay (with eager
    # work and synchronisations between) must give the eager result bit for bit, and a replay
    # after new inputs are copied into the same buffers must give the eager result on them.
    import vision_transformer_attention_amd as vta
    w = inputs.custom([300, 129, 1, 64], n_heads=4, head_dim=80, dtype=inputs.BF16, seed=21)
    q, k, v, cu, scale = inputs.make(w)
    d = torch.device("cuda:0")
    qd, kd, vd, cud = q.to(d), k.to(d), v.to(d), cu.to(d)
    out = torch.empty_like(qd)
    vta.fwd(qd, kd, vd, cud, scale, out=out, check_cu=False, causal=causal)  # device set-up, outside the graph
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vta.fwd(qd, kd, vd, cud, scale, out=out, check_cu=False, causal=causal)
    torch.cuda.synchronize()
    for i in range(3):
        say(f"graph replay {i} (causal={causal})")
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
    q2, k2, v2, _, _ = inputs.make(inputs.custom([300, 129, 1, 64], n_heads=4, head_dim=80, dtype=inputs.BF16,
                                                 seed=22))
    qd.copy_(q2.to(d))
    kd.copy_(k2.to(d))
    vd.copy_(v2.to(d))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    fresh = vta.fwd(q2.to(d), k2.to(d), v2.to(d), cud, scale, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(out, fresh)
    assert not torch.equal(out, eager)


def test_empty_batch_is_a_noop():
    d = torch.device("cuda:0")
    q = torch.zeros(0, 2, 64, dtype=torch.bfloat16, device=d)
    o = __import__("vision_transformer_attention_amd").fwd(q, q, q, torch.zeros(1, dtype=torch.int32, device=d))
    assert o.shape == q.shape


def test_packed_equals_each_image_alone_bitwise():
    w = inputs.custom([300, 1, 129, 64, 513], n_heads=4, head_dim=80, dtype=inputs.BF16, seed=13)
    q, k, v, cu, scale = inputs.make(w)
    packed = run_gpu(q, k, v, cu, scale)
    c = cu.numpy()
    for s in range(len(c) - 1):
        a, b = int(c[s]), int(c[s + 1])
        alone = run_gpu(q[a:b].contiguous(), k[a:b].contiguous(), v[a:b].contiguous(),
                        torch.tensor([0, b - a], dtype=torch.int32), scale)
        assert torch.equal(alone, packed[a:b]), s


def test_head_independence_bitwise():
    w = inputs.custom([200, 77], n_heads=3, head_dim=64, dtype=inputs.BF16, seed=14)
    q, k, v, cu, scale = inputs.make(w)
    base = run_gpu(q, k, v, cu, scale)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[:, 1] = -q2[:, 1]
    k2[:, 1] = k2[:, 1] * 2
    v2[:, 1] = v2[:, 1] + 1
    got = run_gpu(q2, k2, v2, cu, scale)
    assert torch.equal(got[:, 0], base[:, 0]) and torch.equal(got[:, 2], base[:, 2])


@pytest.mark.parametrize("name", ["page-912", "packed-varlen-8", "f32-mixed", "long-16384", "packed-window-256",
                                  "mid-2000"])
def test_deterministic_bitwise(name):
    # The launch has a fixed schedule (no atomics, no order-dependent reductions), so any
    # run-to-run difference means a race: an LDS buffer reused too early, or a register
    # overwritten while an in-flight matrix instruction still reads it.  page-912 runs the
    # short-image items split by keys between wavefront pairs, packed-varlen-8 the 256-query
    # ones; long-16384 (head_dim 128), the narrow window and a 2000-token image (64-query
    # items) run the steps that read their V^T operands before the score products.
    window = 0
    if name == "f32-mixed":
        w = inputs.custom([700, 300, 45], n_heads=4, head_dim=80, dtype=inputs.F32, seed=31)
    elif name == "packed-window-256":
        w, window = inputs.WORKLOADS["packed-varlen-8"], 256
    elif name == "mid-2000":
        w = inputs.custom([2000], n_heads=16, head_dim=80, dtype=inputs.BF16, seed=32)
    else:
        w = inputs.WORKLOADS[name]
    say(f"[determinism] {name}")
    q, k, v, cu, scale = inputs.make(w)
    d = torch.device("cuda:0")
    qd, kd, vd, cud = q.to(d), k.to(d), v.to(d), cu.to(d)
    import vision_transformer_attention_amd as vta
    first = vta.fwd(qd, kd, vd, cud, scale, window=window)
    for _ in range(4):
        again = vta.fwd(qd, kd, vd, cud, scale, window=window)
        assert torch.equal(first, again)
    torch.cuda.synchronize()


def test_non_default_stream_and_no_host_sync_needed():
    w = inputs.custom([500, 33], n_heads=2, head_dim=128, dtype=inputs.BF16, seed=15)
    q, k, v, cu, scale = inputs.make(w)
    s = torch.cuda.Stream()
    o = run_gpu(q, k, v, cu, scale, stream=s)
    ref = oracle.attention(q, k, v, cu, scale)
    err = float(np.max(np.abs(o.float().numpy() - ref)))
    say(f"[parity] non-default stream: max-abs err {err:.3e}")
    assert err <= TOL[inputs.BF16]


def test_concurrent_streams_match_sequential_bitwise():
    # launches on two streams at once (no host sync between them) give the results of the
    # same launches one after the other: the library keeps no per-call state on the device
    import vision_transformer_attention_amd as vta
    dev = torch.device("cuda:0")
    cases = []
    for w, kw in ((inputs.WORKLOADS["page-912"], {}), (inputs.custom([700, 64, 1, 300], n_heads=8, head_dim=64,
                                                                      dtype=inputs.BF16, seed=17, n_kv_heads=2),
                                                       {"causal": True})):
        q, k, v, cu, scale = inputs.make(w)
        cases.append(([x.to(dev) for x in (q, k, v, cu)], scale, kw))
    seq = []
    for (q, k, v, cu), scale, kw in cases:
        seq.append(vta.fwd(q, k, v, cu, scale, **kw))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(c[0][0]) for c in cases]
    for _ in range(20):  # many launches in flight on both streams
        for st, ((q, k, v, cu), scale, kw), o in zip(streams, cases, outs):
            with torch.cuda.stream(st):
                vta.fwd(q, k, v, cu, scale, out=o, check_cu=False, **kw)
    torch.cuda.synchronize()
    for a, b in zip(seq, outs):
        assert torch.equal(a, b)


def test_constant_v_gives_constant_output():
    w = inputs.custom([1000], n_heads=2, head_dim=80, dtype=inputs.BF16, seed=16)
    q, k, v, cu, scale = inputs.make(w)
    v = torch.full_like(v, 1.5)
    o = run_gpu(q, k, v, cu, scale)
    assert float((o.float() - 1.5).abs().max()) <= 1e-2


# ---- grouped-query attention (K/V with a divisor of the query heads) ----

@pytest.mark.parametrize("dtype,head_dim,h,hkv", [(inputs.BF16, 64, 8, 2), (inputs.BF16, 72, 6, 3),
                                                  (inputs.BF16, 80, 8, 1), (inputs.BF16, 128, 8, 4),
                                                  (inputs.F32, 64, 4, 2), (inputs.F32, 80, 6, 1)])
def test_grouped_query_edge_lengths(dtype, head_dim, h, hkv):
    lengths = [1, 31, 64, 65, 129, 300]
    w = inputs.custom(lengths, n_heads=h, head_dim=head_dim, dtype=dtype, seed=200 + head_dim + hkv, n_kv_heads=hkv)
    check_workload(w, full=True)


def test_grouped_query_rising_scores():
    w = inputs.custom([1000, 64, 5], n_heads=8, head_dim=80, dtype=inputs.BF16, seed=29, key_ramp=300.0, spikes=2,
                      n_kv_heads=2)
    check_workload(w, full=True)


def test_grouped_query_packed_sampled_rows():
    check_workload(inputs.WORKLOADS["packed-varlen-8-gqa4"], full=False)


@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.F32])
def test_grouped_query_equals_repeated_kv_bitwise(dtype):
    # reading K/V head h // g in place gives bitwise the multi-head result on K/V widened by copying
    w = inputs.custom([300, 77, 1000, 1], n_heads=8, head_dim=80, dtype=dtype, seed=30, n_kv_heads=2)
    q, k, v, cu, scale = inputs.make(w)
    say(f"[parity] gqa vs repeated kv: {w.lengths} H=8 Hkv=2 {dtype}")
    o_gqa = run_gpu(q, k, v, cu, scale)
    o_mha = run_gpu(q, k.repeat_interleave(4, dim=1).contiguous(), v.repeat_interleave(4, dim=1).contiguous(), cu,
                    scale)
    assert torch.equal(o_gqa, o_mha)


# ---- half inputs, and float32 outputs from 16-bit inputs ----

@pytest.mark.parametrize("head_dim", [64, 72, 80, 128])
def test_half_edge_lengths(head_dim):
    lengths = [1, 2, 31, 32, 33, 63, 64, 65, 127, 129, 300]
    w = inputs.custom(lengths, n_heads=3, head_dim=head_dim, dtype=inputs.F16, seed=300 + head_dim)
    check_workload(w, full=True)


@pytest.mark.parametrize("head_dim", [80, 128])
def test_half_rising_and_jumping_scores(head_dim):
    # half keeps its weights in [2^-14 .., 2^15): the raise path runs whenever a score climbs
    # 15 log2 units past the offset, many times over these ramps and spikes
    w = inputs.custom([1000, 777, 64, 33, 5], n_heads=2, head_dim=head_dim, dtype=inputs.F16, seed=31,
                      key_ramp=300.0, spikes=2)
    check_workload(w, full=True)


def test_half_page_912():
    w = inputs.custom([912], n_heads=16, head_dim=80, dtype=inputs.F16, seed=32, token_factor=(0.5, 2.0))
    check_workload(w, full=True)


@pytest.mark.parametrize("dtype,head_dim", [(inputs.BF16, 80), (inputs.BF16, 128), (inputs.F16, 64),
                                             (inputs.F16, 72)])
def test_float32_output_from_16_bit_inputs(dtype, head_dim):
    w = inputs.custom([1, 65, 300, 129], n_heads=3, head_dim=head_dim, dtype=dtype, seed=33 + head_dim)
    o32, _ = check_workload(w, full=True, out_dtype=torch.float32)
    # the 16-bit output is the float32 one rounded to nearest even, bit for bit
    q, k, v, cu, scale = inputs.make(w)
    o16 = run_gpu(q, k, v, cu, scale)
    assert torch.equal(o32.to(o16.dtype), o16)


def test_float32_output_grouped_query_packed_sampled():
    check_workload(inputs.WORKLOADS["packed-varlen-8-gqa4"], full=False, out_dtype=torch.float32)


@pytest.mark.gpu
@pytest.mark.parametrize("extra", [1, 9, 257, 263])
def test_large_item_deal_around_one_round_of_the_grid(extra):
    # Launches with more large items than one round of the grid are dealt in tiers of half the
    # grid, alternately to the two halves of the CU pairs; G + extra items (one head, so an item
    # is one 256-query block of an image) with every item checked at two rows.
    from vision_transformer_attention_amd import binding
    cfg = binding.kernel_config(80, torch.bfloat16)
    grid, bm = cfg["grid"], cfg["block_m"]
    rng = np.random.default_rng(500 + extra)
    target = grid + extra
    blocks = []
    while sum(blocks) < target:
        blocks.append(int(min(rng.integers(8, 40), target - sum(blocks))))
    lengths = [b * bm - int(rng.integers(0, bm - 1)) for b in blocks]  # ragged last blocks
    assert sum(-(-n // bm) for n in lengths) == target
    w = inputs.custom(lengths, n_heads=1, head_dim=80, dtype=inputs.BF16, seed=77 + extra)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    rows = []
    for s, n in enumerate(lengths):
        for b in range(-(-n // bm)):
            for off in ((7 * b) % 64, bm // 2 + (13 * b) % 64):
                r = min(b * bm + off, n - 1)
                rows.append(int(cu[s]) + r)
    check_workload(w, full=False, rows=np.array(sorted(set(rows)), np.int64))
