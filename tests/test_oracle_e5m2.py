"""Pins of the oracle's E5M2 decoding (CPU only)."""
import math
import os

import numpy as np
import torch

from oracle import decode_e5m2_byte, decode_e5m2_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e5m2_known_values.txt")


def test_all_bytes_match_torch_float8_e5m2():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
    tab = decode_e5m2_table()
    nan = np.isnan(ref)
    assert (np.isnan(tab) == nan).all()
    assert np.array_equal(tab[~nan], ref[~nan])             # infinities included
    assert np.array_equal(np.signbit(tab[~nan]), np.signbit(ref[~nan]))


def test_hand_listed_values_of_the_format():
    n = 0
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            byte, val = line.split()
            v = decode_e5m2_byte(int(byte, 16))
            want = float(val)
            if math.isnan(want):
                assert math.isnan(v), byte
            else:
                assert v == want and math.copysign(1, v) == math.copysign(1, want), (byte, v, want)
            n += 1
    assert n >= 20


def test_specials_sit_at_exponent_31():
    tab = decode_e5m2_table()
    assert set(np.flatnonzero(np.isnan(tab)).tolist()) == {0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF}
    assert set(np.flatnonzero(np.isinf(tab)).tolist()) == {0x7C, 0xFC}


def test_sign_symmetry_and_order():
    tab = decode_e5m2_table()
    for b in range(0x7D):
        assert tab[b | 0x80] == -tab[b]
    fin = tab[:0x7C]
    assert (np.diff(fin) > 0).all()           # strictly increasing magnitudes 0x00..0x7B
    assert fin[-1] == 57344.0


def test_every_byte_is_the_upper_byte_of_its_fp16_value():
    # E5M2 shares FP16's sign, exponent width and bias: byte b encodes the FP16 value whose
    # bit pattern is b << 8 (numpy's IEEE binary16, a library routine).
    tab = decode_e5m2_table()
    halves = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    nan = np.isnan(tab)
    assert (np.isnan(halves) == nan).all()
    assert np.array_equal(halves[~nan], tab[~nan])
