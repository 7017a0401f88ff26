"""E5M2 byte decoding, written from the format definition (test infrastructure only).

The pages name E5M2 as one of the KV cache formats the attention backend keeps serving
besides E4M3 ("DFlash2 concurrent long-context attention, 2026-09-27", section "Why the
single-request optimization was missing from concurrent decode"), and "SM70 attention and
quantized projection coverage across TP sizes", section "Additional findings, 2026-09-21
11:40 CST", counts FP16/E5M2 multi-head graph regressions among its checks. They do not
define it; the reading taken here is the OCP 8-bit floating-point E5M2 encoding (IEEE-like,
with infinities):

* bit 7 is the sign,
* bits 6..2 are the exponent field ``e`` with bias 15,
* bits 1..0 are the mantissa field ``m``,
* ``e == 0`` encodes subnormals ``m/4 * 2**(1-15)``,
* ``e == 31`` encodes infinity (``m == 0``) and NaN (``m != 0``); the largest finite
  magnitude is ``1.75 * 2**15 = 57344``.

Pinned by: all 256 bytes against ``torch.float8_e5m2`` widened to float64 (a library
routine), hand-listed values of the format in ``tests/golden``, structural properties
(sign symmetry, monotonic order) and the identity with the upper byte of an FP16 value.
"""
import math

import numpy as np


def decode_byte(b: int) -> float:
    """Value of one E5M2 byte as a Python float (exact; +-inf and NaN where the format says)."""
    if not 0 <= b <= 255:
        raise ValueError(f"not a byte: {b}")
    sign = -1.0 if (b >> 7) & 1 else 1.0
    e = (b >> 2) & 0x1F
    m = b & 0x3
    if e == 0x1F:
        return sign * math.inf if m == 0 else math.nan
    if e == 0:
        return sign * (m / 4.0) * 2.0 ** (1 - 15)
    return sign * (1.0 + m / 4.0) * 2.0 ** (e - 15)


def decode_table() -> np.ndarray:
    """float64[256] with ``table[b] = decode_byte(b)``."""
    return np.array([decode_byte(b) for b in range(256)], dtype=np.float64)
