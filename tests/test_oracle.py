"""The float64 oracle against its pins (closed forms, invariants, a library routine)."""
import numpy as np
import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(lib, pin):
    pin(lib)


def test_empty_batch_and_zero_length_sequences(lib):
    q = np.zeros((0, 2, 4), np.float32)
    out = oracle.attention(q, q, q, [0], 0.5, lib=lib)
    assert out.shape == (0, 2, 4)
    out = oracle.attention(q, q, q, [0, 0, 0], 0.5, lib=lib)
    assert out.shape == (0, 2, 4)


def test_rejects_bad_cu_seqlens(lib):
    q = np.zeros((4, 1, 2), np.float32)
    for cu in ([1, 4], [0, 3], [0, 3, 2, 4]):
        with pytest.raises(ValueError):
            oracle.attention(q, q, q, cu, 1.0, lib=lib)
    with pytest.raises(RuntimeError):
        oracle.attention_rows(q, q, q, [0, 4], 1.0, [4], lib=lib)


def test_threads_reported(lib):
    assert oracle.threads() >= 1
