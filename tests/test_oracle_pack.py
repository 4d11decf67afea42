"""Pins for the packing format, the order of the codes inside every 8 and
the tiled storage order: hand-worked words and indices, round trips,
bijection."""
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


def test_tiled_index_worked(golden_dir):
    with open(os.path.join(golden_dir, "tiled_layout.json")) as f:
        g = json.load(f)
    for c in g["codes"]:
        assert int(oracle.tiled_code_index(c["n"], c["b"], c["w"], c["q"], c["d"])) == c["index"], c
    for c in g["groups"]:
        v = np.zeros((c["d_out"], c["ng"]), np.float32)
        v[c["n"], c["gi"]] = 1.0
        assert int(np.argmax(oracle.tile_groups(v))) == c["index"]


@pytest.mark.parametrize("q", [2, 3, 4, 5])
def test_tiled_layout_is_a_bijection(q):
    d_out, d = 96, 320
    n, b, w = np.meshgrid(np.arange(d_out), np.arange(d // 32), np.arange(q), indexing="ij")
    idx = oracle.tiled_code_index(n, b, w, q, d).ravel()
    assert np.array_equal(np.sort(idx), np.arange(d_out * d // 32 * q))
    words = np.random.default_rng(q).integers(0, 2 ** 32, size=(d_out, d // 32, q), dtype=np.uint64).astype(np.uint32)
    np.testing.assert_array_equal(oracle.untile_codes(oracle.tile_codes(words, q), q, d_out, d), words)
    vals = np.random.default_rng(q).standard_normal((d_out, d // 32)).astype(np.float16)
    np.testing.assert_array_equal(oracle.untile_groups(oracle.tile_groups(vals), d_out, d // 32), vals)


def test_tiled_step_chunks_are_contiguous():
    # one 64-channel step of one 32-row tile occupies one contiguous run of 32*2q words
    q, d_out, d = 4, 64, 256
    n, b, w = np.meshgrid(np.arange(32, 64), np.array([4, 5]), np.arange(q), indexing="ij")
    idx = np.sort(oracle.tiled_code_index(n, b, w, q, d).ravel())
    assert np.array_equal(idx, np.arange(idx[0], idx[0] + 32 * 2 * q))
    # and a row's step words put the words of MFMA lane half 0 (w = 0, 2) first
    row = oracle.tiled_code_index(5, np.array([0, 0, 1, 1, 0, 0, 1, 1]), np.array([0, 2, 0, 2, 1, 3, 1, 3]), 4, d)
    assert np.array_equal(row - row[0], np.arange(8))


def test_slot_order_worked_words(golden_dir):
    with open(os.path.join(golden_dir, "slot_order.json")) as f:
        g = json.load(f)
    for q, words in g["words"].items():
        q = int(q)
        codes = (np.arange(32) % (1 << q)).astype(np.uint8)[None, :]
        packed = oracle.pack(oracle.interleave8(codes), q)
        assert [hex(int(w)) for w in packed[0, 0]] == words


def test_slot_order_pairs_natural_channels():
    # slots j and j + 4 of every group of 8 hold channels 2j and 2j + 1
    ch = np.arange(64)[None, :]
    st8 = oracle.interleave8(ch).reshape(8, 8)
    for grp in range(8):
        for j in range(4):
            assert st8[grp, j] == 8 * grp + 2 * j and st8[grp, j + 4] == 8 * grp + 2 * j + 1


@pytest.mark.parametrize("q", [2, 3, 4, 5])
def test_device_codes_roundtrip(q):
    d_out, d = 64, 192
    codes = np.random.default_rng(10 + q).integers(0, 1 << q, size=(d_out, d)).astype(np.uint8)
    np.testing.assert_array_equal(oracle.deinterleave8(oracle.interleave8(codes)), codes)
    flat = oracle.device_codes(codes, q)
    assert flat.dtype == np.uint32 and flat.size == d_out * d // 32 * q
    np.testing.assert_array_equal(oracle.codes_from_device(flat, q, d_out, d), codes)
