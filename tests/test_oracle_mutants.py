"""Plant plausible slips in a copy of the oracle's C source and check that the pins catch each.

Mistakes are planted only in a temporary copy of the oracle, compiled and run on
the CPU in a child process (so a mutant that crashes cannot take pytest down; a
crash also counts as caught).
"""
import os
import subprocess
import sys

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "vitattn_ref.c")
TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)

MUTANTS = {
    "exp-sign": [("exp(w[j - a] - m)", "exp(m - w[j - a])")],
    "scale-dropped": [("double logit = scale * dot;", "double logit = dot;")],
    "value-is-key": [("const float* vj = v + ", "const float* vj = k + ")],
    "query-head-ignored": [("const float* qi = q + i * row_stride + (int64_t)h * head_dim;",
                            "const float* qi = q + i * row_stride;")],
    "key-head-ignored": [("const float* kj = k + j * kv_stride + (int64_t)hk * head_dim;\n    double dot",
                          "const float* kj = k + j * kv_stride;\n    double dot")],
    "kv-head-modulo": [("const int32_t hk = h / (n_heads / n_kv_heads);",
                        "const int32_t hk = h % n_kv_heads;")],
    "kv-stride-is-query-stride": [("const int64_t kv_stride = (int64_t)n_kv_heads * head_dim;",
                                   "const int64_t kv_stride = (int64_t)n_heads * head_dim;")],
    "no-normalisation": [("for (int32_t e = 0; e < head_dim; ++e) out[e] /= z;",
                          "for (int32_t e = 0; e < head_dim; ++e) out[e] /= 1.0;")],
    "keys-cross-images": [
        ("double* w = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));",
         "double* w = (double*)malloc(sizeof(double) * (size_t)(cu_seqlens[n_seqs] + 1));"),
        ("ref_one_row(q, k, v, a, b, i, h, n_heads, n_kv_heads, head_dim, scale, causal, window, w,",
         "ref_one_row(q, k, v, 0, cu_seqlens[n_seqs], i, h, n_heads, n_kv_heads, head_dim, scale, causal, window, w,"),
    ],
    "last-key-dropped": [("for (int64_t j = a; j < b; ++j) {\n    if (!ref_visible",
                          "for (int64_t j = a; j < b - 1; ++j) {\n    if (!ref_visible")],
    "max-subtracted-from-one-key": [("exp(w[j - a] - m)", "exp(w[j - a] - (j == a ? m : 0.0))")],
    "sum-misses-first-key": [("    z += wj;\n", "    if (j > a) z += wj;\n")],
    "causal-ignored": [("if (causal && kj > qi + (lk - lq)) return 0;", "if (0 && kj > qi + (lk - lq)) return 0;")],
    "causal-flipped": [("if (causal && kj > qi + (lk - lq)) return 0;", "if (causal && kj < qi + (lk - lq)) return 0;")],
    "causal-one-ahead": [("if (causal && kj > qi + (lk - lq)) return 0;",
                          "if (causal && kj > qi + 1 + (lk - lq)) return 0;")],
    "causal-drops-diagonal": [("if (causal && kj > qi + (lk - lq)) return 0;",
                               "if (causal && kj >= qi + (lk - lq)) return 0;")],
    "window-inclusive": [("if (window > 0 && (qi - kj >= window || kj - qi >= window)) return 0;",
                          "if (window > 0 && (qi - kj > window || kj - qi > window)) return 0;")],
    "window-one-sided": [("if (window > 0 && (qi - kj >= window || kj - qi >= window)) return 0;",
                          "if (window > 0 && (qi - kj >= window)) return 0;")],
    "window-ignored-with-causal": [("if (window > 0 && (qi - kj >= window",
                                    "if (window > 0 && !causal && (qi - kj >= window")],
    "window-ignored": [("if (window > 0 && (qi - kj >= window", "if (0 && (qi - kj >= window")],
    "window-from-image-start": [("if (window > 0 && (qi - kj >= window || kj - qi >= window)) return 0;",
                                 "if (window > 0 && (kj >= window)) return 0;")],
    "prologue-rotate-half-sign": [("const double rot = d < h ? -y[d + h] : y[d - h];",
                                   "const double rot = d < h ? y[d + h] : -y[d - h];")],
    "prologue-interleaved-pairs": [("const double rot = d < h ? -y[d + h] : y[d - h];",
                                    "const double rot = d % 2 == 0 ? -y[d + 1] : y[d - 1];")],
    "prologue-cos-sin-swapped": [("out[d] = y[d] * (double)cosr[d] + rot * (double)sinr[d];",
                                  "out[d] = y[d] * (double)sinr[d] + rot * (double)cosr[d];")],
    "prologue-eps-outside-sqrt": [("const double r = 1.0 / sqrt(ms + eps);",
                                   "const double r = 1.0 / (sqrt(ms) + eps);")],
    "prologue-sum-not-mean": [("    ms /= (double)D;\n", "")],
    "prologue-gain-ignored": [("y[d] = y[d] * r * (double)w[d];", "y[d] = y[d] * r;")],
    "prologue-k-takes-q-gain": [("ref_norm_rope(row + (H + h) * D, c, s, kw,", "ref_norm_rope(row + (H + h) * D, c, s, qw,")],
    "prologue-v-from-k-slot": [("v[(t * G + h) * D + d] = (double)row[(H + G + h) * D + d];",
                                "v[(t * G + h) * D + d] = (double)row[(H + h) * D + d];")],
    "prologue-k-slot-after-q-of-kv-width": [("ref_norm_rope(row + (H + h) * D, c, s, kw,",
                                            "ref_norm_rope(row + (G + h) * D, c, s, kw,")],
    "value-head-ignored": [("const float* vj = v + j * kv_stride + (int64_t)hk * head_dim;",
                            "const float* vj = v + j * kv_stride;")],
}

RUNNER = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle
from oracle_pins import PINS
lib = oracle.load({lib!r})
caught = []
for pin in PINS:
    try:
        pin(lib)
    except (AssertionError, RuntimeError):
        caught.append(pin.__name__)
print("CAUGHT", ",".join(caught))
"""


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(tmp_path, name):
    with open(SRC) as f:
        text = f.read()
    for old, new in MUTANTS[name]:
        assert text.count(old) >= 1, f"mutation anchor for {name} not found: {old!r}"
        text = text.replace(old, new, 1)
    src = tmp_path / "vitattn_ref.c"
    src.write_text(text)
    lib_path = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", str(src), "-lm", "-o", lib_path], check=True)
    code = RUNNER.format(root=ROOT, tests=TESTS, lib=lib_path)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return  # the mutant crashed or raised: caught
    line = [l for l in r.stdout.splitlines() if l.startswith("CAUGHT")][-1]
    caught = [c for c in line[len("CAUGHT"):].strip().split(",") if c]
    assert caught, f"no pin caught the planted mistake {name}"
