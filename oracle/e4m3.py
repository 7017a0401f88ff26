"""E4M3 byte decoding, written from the format definition (test infrastructure only).

The pages name the KV format only as "E4M3" (DFlash2 long-batch design note,
"Why the single-request optimization was missing from concurrent decode"; SM70
TP shape coverage, "Implementation and validation in progress", which tests all
byte encodings of the exact conversion). The reading taken here is the OCP 8-bit
floating-point E4M3 encoding without infinities (often called E4M3FN):

* bit 7 is the sign,
* bits 6..3 are the exponent field ``e`` with bias 7,
* bits 2..0 are the mantissa field ``m``,
* ``e == 0`` encodes subnormals ``m/8 * 2**(1-7)``,
* ``e == 15, m == 7`` (bytes 0x7F and 0xFF) is NaN; there is no infinity,
  so the largest finite magnitude is ``1.75 * 2**8 = 448``.

Pinned by: all 256 bytes against ``torch.float8_e4m3fn`` widened to float64 (a
library routine), hand-listed values of the format in ``tests/golden``, and
structural properties (sign symmetry, monotonic order, exact FP16
representability).
"""
import math

import numpy as np


def decode_byte(b: int) -> float:
    """Value of one E4M3 byte as a Python float (exact; NaN for 0x7F/0xFF)."""
    if not 0 <= b <= 255:
        raise ValueError(f"not a byte: {b}")
    sign = -1.0 if (b >> 7) & 1 else 1.0
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def decode_table() -> np.ndarray:
    """float64[256] with ``table[b] = decode_byte(b)``."""
    return np.array([decode_byte(b) for b in range(256)], dtype=np.float64)
