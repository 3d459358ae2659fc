"""The C ABI library on the CPU: it loads, exports what include/vitattn.h declares,
and rejects bad arguments before making any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import vision_transformer_attention_amd as vta
from vision_transformer_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vitattn.h")

OK, INVALID, BAD_HD, BAD_DT, NO_DEV, OOM, HIPERR = 0, -1, -2, -3, -4, -5, -6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vitattn_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return vta.load_library()


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(
        ["vitattn_fwd", "vitattn_fwd_gqa", "vitattn_fwd_masked", "vitattn_qkv_prologue", "vitattn_status_string",
         "vitattn_last_error", "vitattn_kernel_config"])


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(binding.library_path())
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_library_is_gfx950_code_object():
    data = open(binding.library_path(), "rb").read()
    assert b"gfx950" in data


def test_status_strings_cover_every_code(lib):
    seen = set()
    for code in (OK, INVALID, BAD_HD, BAD_DT, NO_DEV, OOM, HIPERR):
        s = lib.vitattn_status_string(code)
        assert s and s != b"unknown status"
        seen.add(s)
    assert len(seen) == 7
    assert lib.vitattn_status_string(12345) == b"unknown status"


FAKE = 0x10000  # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("args,status", [
    (dict(n_seqs=-1), INVALID),
    (dict(n_heads=0), INVALID),
    (dict(n_heads=-3), INVALID),
    (dict(head_dim=96), BAD_HD),
    (dict(head_dim=0), BAD_HD),
    (dict(dtype=5), BAD_DT),
    (dict(dtype=-1), BAD_DT),
    (dict(dtype=2, head_dim=96), BAD_HD),   # f16: a known dtype, so the head_dim is what fails
    (dict(dtype=3, head_dim=96), BAD_HD),   # bf16 in, f32 out
    (dict(dtype=4, head_dim=96), BAD_HD),   # f16 in, f32 out
    (dict(dtype=4, n_seqs=0), OK),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(q=0), INVALID),
    (dict(o=0), INVALID),
    (dict(cu=0), INVALID),
    (dict(q=FAKE + 8), INVALID),        # misaligned
    (dict(cu=FAKE + 2), INVALID),       # misaligned
    (dict(n_seqs=0), OK),               # nothing to do: no HIP call at all
    (dict(n_seqs=0, q=0, k=0, v=0, o=0, cu=0), OK),
])
def test_validation_before_any_hip_call(lib, args, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, cu=FAKE, n_seqs=1, n_heads=2, head_dim=80, scale=0.1, dtype=1)
    a.update(args)
    rc = lib.vitattn_fwd(a["q"], a["k"], a["v"], a["o"], a["cu"], a["n_seqs"], a["n_heads"], a["head_dim"],
                         ctypes.c_float(a["scale"]), a["dtype"], None)
    assert rc == status
    if status != OK:
        assert len(lib.vitattn_last_error()) > 0


@pytest.mark.parametrize("args,status", [
    (dict(n_kv_heads=0), INVALID),
    (dict(n_kv_heads=-1), INVALID),
    (dict(n_kv_heads=3), INVALID),      # not a divisor of 8 query heads
    (dict(n_kv_heads=16), INVALID),     # more K/V heads than query heads
    (dict(n_kv_heads=2, head_dim=96), BAD_HD),
    (dict(n_kv_heads=2, q=FAKE + 4), INVALID),
    (dict(n_kv_heads=2, n_seqs=0), OK),
])
def test_gqa_validation_before_any_hip_call(lib, args, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, cu=FAKE, n_seqs=1, n_heads=8, n_kv_heads=2, head_dim=80, scale=0.1,
             dtype=1)
    a.update(args)
    rc = lib.vitattn_fwd_gqa(a["q"], a["k"], a["v"], a["o"], a["cu"], a["n_seqs"], a["n_heads"], a["n_kv_heads"],
                             a["head_dim"], ctypes.c_float(a["scale"]), a["dtype"], None)
    assert rc == status
    if status != OK:
        assert len(lib.vitattn_last_error()) > 0


@pytest.mark.parametrize("args,status", [
    (dict(causal=2), INVALID),
    (dict(causal=-1), INVALID),
    (dict(window=-1), INVALID),
    (dict(window=-(2 ** 31)), INVALID),
    (dict(causal=1, n_kv_heads=3), INVALID),   # the grouped-query checks still apply
    (dict(causal=1, head_dim=96), BAD_HD),
    (dict(window=4, dtype=7), BAD_DT),
    (dict(causal=1, scale=float("nan")), INVALID),
    (dict(causal=1, cu=FAKE + 1), INVALID),
    (dict(causal=1, window=5, n_seqs=0), OK),
    (dict(causal=2, n_seqs=0), INVALID),       # a bad mask is an error even with nothing to do
])
def test_masked_validation_before_any_hip_call(lib, args, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, cu=FAKE, n_seqs=1, n_heads=8, n_kv_heads=2, head_dim=80, scale=0.1,
             causal=0, window=0, dtype=1)
    a.update(args)
    rc = lib.vitattn_fwd_masked(a["q"], a["k"], a["v"], a["o"], a["cu"], a["n_seqs"], a["n_heads"],
                                a["n_kv_heads"], a["head_dim"], ctypes.c_float(a["scale"]), a["causal"],
                                a["window"], a["dtype"], None)
    assert rc == status
    if status != OK:
        assert len(lib.vitattn_last_error()) > 0


@pytest.mark.parametrize("args,status", [
    (dict(n_tokens=-1), INVALID),
    (dict(n_heads=0), INVALID),
    (dict(n_kv_heads=3), INVALID),
    (dict(head_dim=96), BAD_HD),
    (dict(head_dim=0), BAD_HD),
    (dict(dtype=3), BAD_DT),            # the prologue writes its input kind: no float32-output codes
    (dict(dtype=5), BAD_DT),
    (dict(cos=0), INVALID),             # one rope table without the other
    (dict(qw=0), INVALID),              # one gain without the other
    (dict(eps=float("nan")), INVALID),
    (dict(eps=-1.0), INVALID),
    (dict(qkv=0), INVALID),
    (dict(q=FAKE + 4), INVALID),        # 16-byte alignment
    (dict(v=FAKE + 8), INVALID),
    (dict(dtype=0, k=FAKE + 8), INVALID),
    (dict(cos=FAKE + 8, sin=FAKE + 8), INVALID),
    (dict(cos=0, sin=0, qw=0, kw=0, eps=float("nan"), n_tokens=0), OK),  # no norm: eps unused
    (dict(n_tokens=0), OK),
    (dict(n_tokens=0, qkv=0, q=0, k=0, v=0), OK),
])
def test_prologue_validation_before_any_hip_call(lib, args, status):
    a = dict(qkv=FAKE, cos=FAKE, sin=FAKE, qw=FAKE, kw=FAKE, eps=1e-6, q=FAKE, k=FAKE, v=FAKE, n_tokens=4,
             n_heads=8, n_kv_heads=2, head_dim=80, dtype=1)
    a.update(args)
    nul = lambda x: x if x else None
    rc = lib.vitattn_qkv_prologue(nul(a["qkv"]), nul(a["cos"]), nul(a["sin"]), nul(a["qw"]), nul(a["kw"]),
                                  ctypes.c_float(a["eps"]), nul(a["q"]), nul(a["k"]), nul(a["v"]), a["n_tokens"],
                                  a["n_heads"], a["n_kv_heads"], a["head_dim"], a["dtype"], None)
    assert rc == status
    if status != OK:
        assert len(lib.vitattn_last_error()) > 0


def test_kernel_config_validates(lib):
    x = ctypes.c_int32(0)
    assert lib.vitattn_kernel_config(96, 1, ctypes.byref(x), None, None, None) == BAD_HD
    assert lib.vitattn_kernel_config(80, 5, None, None, None, None) == BAD_DT
    assert lib.vitattn_kernel_config(72, 4, None, None, None, None) != BAD_DT


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_present(), reason="checks the no-device path; a GPU is present")
def test_no_device_is_reported_not_faked(lib):
    rc = lib.vitattn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 80, ctypes.c_float(0.1), 1, None)
    assert rc == NO_DEV
    assert lib.vitattn_kernel_config(80, 1, None, None, None, None) == NO_DEV


def test_binding_checks_cu_seqlens():
    binding.check_cu_seqlens(np.array([0, 3, 3, 10], np.int32), 10)
    for bad, t in (([1, 10], 10), ([0, 5, 4, 10], 10), ([0, 9], 10), ([], 0)):
        with pytest.raises(ValueError):
            binding.check_cu_seqlens(np.array(bad, np.int32), t)


def test_binding_rejects_cpu_and_bad_tensors():
    import torch
    q = torch.zeros(4, 2, 80, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        vta.fwd(q, q, q, cu)  # CPU tensors: the library never computes on the CPU
    with pytest.raises(TypeError):
        vta.fwd(q.float().numpy(), q, q, cu)


def test_binding_dtype_codes():
    import torch
    from vision_transformer_attention_amd import binding as b
    assert b._call_code(torch.float32, torch.float32) == 0
    assert b._call_code(torch.bfloat16, torch.bfloat16) == 1
    assert b._call_code(torch.float16, torch.float16) == 2
    assert b._call_code(torch.bfloat16, torch.float32) == 3
    assert b._call_code(torch.float16, torch.float32) == 4
    for bad in ((torch.float32, torch.bfloat16), (torch.bfloat16, torch.float16), (torch.float16, torch.bfloat16)):
        with pytest.raises(TypeError):
            b._call_code(*bad)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    # no CPU fallback: without the HIP library every entry point of the binding raises
    import torch
    with pytest.raises(binding.VitattnError):
        binding.load_library(str(tmp_path / "libvitattn.so"))
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "library_path", lambda: str(tmp_path / "libvitattn.so"))
    q = torch.zeros(4, 2, 80, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(binding.VitattnError):
        vta.fwd(q, q, q, cu)
