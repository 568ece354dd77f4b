"""Pins of the packing oracle: the worked example of the varlen page, a
hand-written case, and the round trip (CPU only)."""

import json
import os

import numpy as np
import pytest

from oracle import pack as P

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_offsets_and_rows():
    g = json.load(open(os.path.join(GOLD, "cu_seqlens_example.json")))
    lengths = g["lengths"]                       # [512, 300, 128]
    assert P.cu_seqlens_from_lengths(lengths).tolist() == g["cu_seqlens"]
    S = max(lengths)
    padded = np.arange(len(lengths) * S, dtype=np.int64).reshape(len(lengths), S)
    packed = P.pack(padded, lengths)
    assert packed.shape == (g["cu_seqlens"][-1],)
    # sequence 1 starts at row 512 and holds padded[1, :300]
    assert packed[512] == S and packed[811] == S + 299 and packed[812] == 2 * S


def test_hand_written_case():
    padded = np.array([[[1, 2], [3, 4], [5, 6]],
                       [[7, 8], [9, 10], [11, 12]],
                       [[13, 14], [15, 16], [17, 18]]], dtype=np.int32)
    packed = P.pack(padded, [2, 0, 3])
    assert packed.tolist() == [[1, 2], [3, 4], [13, 14], [15, 16], [17, 18]]
    back = P.unpack(packed, [0, 2, 2, 5], 3)
    assert back.tolist() == [[[1, 2], [3, 4], [0, 0]],
                             [[0, 0], [0, 0], [0, 0]],
                             [[13, 14], [15, 16], [17, 18]]]


def test_round_trip_and_padding_zeroed():
    rng = np.random.default_rng(5)
    lengths = [0, 7, 1, 16, 16, 3]
    padded = rng.normal(size=(6, 16, 2, 3))
    packed = P.pack(padded, lengths)
    assert packed.shape[0] == sum(lengths)
    back = P.unpack(packed, P.cu_seqlens_from_lengths(lengths), 16)
    for b, n in enumerate(lengths):
        np.testing.assert_array_equal(back[b, :n], padded[b, :n])
        assert np.all(back[b, n:] == 0)
    np.testing.assert_array_equal(P.pack(back, lengths), packed)


def test_rejects_lengths_outside_the_buffer():
    with pytest.raises(ValueError):
        P.pack(np.zeros((2, 4)), [5, 1])
    with pytest.raises(ValueError):
        P.unpack(np.zeros((9, 2)), [0, 9], 4)
