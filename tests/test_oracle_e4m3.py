"""Pins of the oracle's E4M3 decoding (CPU only)."""
import math
import os

import numpy as np
import torch

from oracle import decode_byte, decode_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_known_values.txt")


def test_all_bytes_match_torch_float8_e4m3fn():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = decode_table()
    nan = np.isnan(ref)
    assert (np.isnan(tab) == nan).all()
    assert np.array_equal(tab[~nan], ref[~nan])
    # signed zero is part of the format
    assert np.array_equal(np.signbit(tab[~nan]), np.signbit(ref[~nan]))


def test_hand_listed_values_of_the_format():
    n = 0
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            byte, val = line.split()
            v = decode_byte(int(byte, 16))
            want = float(val)
            if math.isnan(want):
                assert math.isnan(v), byte
            else:
                assert v == want and math.copysign(1, v) == math.copysign(1, want), (byte, v, want)
            n += 1
    assert n >= 20


def test_nan_only_at_s1111111():
    tab = decode_table()
    assert set(np.flatnonzero(np.isnan(tab)).tolist()) == {0x7F, 0xFF}


def test_sign_symmetry_and_order():
    tab = decode_table()
    for b in range(0x7F):
        assert tab[b | 0x80] == -tab[b]
    pos = tab[:0x7F]
    assert (np.diff(pos) > 0).all()          # strictly increasing magnitudes 0x00..0x7E
    assert pos[-1] == 448.0


def test_every_finite_value_is_exact_in_fp16():
    tab = decode_table()
    fin = tab[~np.isnan(tab)]
    assert np.array_equal(fin.astype(np.float16).astype(np.float64), fin)
