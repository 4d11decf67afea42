"""Pins for the packing format: hand-worked words and the round trip."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def test_worked_words(golden_dir):
    with open(os.path.join(golden_dir, "pack_words.json")) as f:
        g = json.load(f)
    for q, words in g["words"].items():
        q = int(q)
        codes = (np.arange(32) % (1 << q)).astype(np.uint8)[None, :]
        packed = oracle.pack(codes, q)
        assert packed.shape == (1, 1, q)
        assert [hex(int(w)) for w in packed[0, 0]] == words


@pytest.mark.parametrize("q", [2, 3, 4, 5])
def test_single_code_positions(q):
    # one code of all-ones at each position k lands at bits [qk, qk+q)
    for k in range(32):
        codes = np.zeros((1, 32), np.uint8)
        codes[0, k] = (1 << q) - 1
        stream = 0
        for i, w in enumerate(oracle.pack(codes, q)[0, 0]):
            stream |= int(w) << (32 * i)
        assert stream == ((1 << q) - 1) << (q * k)


@settings(max_examples=40, deadline=None)
@given(q=st.sampled_from([2, 3, 4, 5]), rows=st.integers(1, 4), blocks=st.integers(1, 4),
       seed=st.integers(0, 2 ** 31))
def test_roundtrip(q, rows, blocks, seed):
    codes = np.random.default_rng(seed).integers(0, 1 << q, size=(rows, 32 * blocks)).astype(np.uint8)
    np.testing.assert_array_equal(oracle.unpack(oracle.pack(codes, q), q, 32 * blocks), codes)


def test_rejects_oversized_codes():
    with pytest.raises(ValueError):
        oracle.pack(np.full((1, 32), 16, np.uint8), 4)
