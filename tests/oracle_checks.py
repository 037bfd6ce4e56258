"""Independent exact-arithmetic helpers used by the oracle pins.

Pure Python with fractions.Fraction: bits are read one at a time from the
packed bytes and values are built from small integer formulas or from the
page's codebook, so nothing here shares code with ``oracle/``.
"""

from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line)
    return rows


def e2m1_codebook():
    """code (0..15) -> Fraction, from the golden codebook file."""
    mags = {}
    for row in read_golden("e2m1_codebook.txt"):
        c, v = row.split()
        mags[int(c)] = Fraction(v)
    book = {}
    for c in range(8):
        book[c] = mags[c]
        book[c | 8] = -mags[c]
    return book


def code_at(row_bytes, j: int, bits: int) -> int:
    """Code j of a packed row, reading bit (j*bits + i) one at a time."""
    v = 0
    for i in range(bits):
        p = j * bits + i
        bit = (int(row_bytes[p // 8]) >> (p % 8)) & 1
        v |= bit << i
    return v


def frac_of_storage(a, dtype: str):
    """Exact Fraction values of stored T data (nested lists)."""
    arr = np.asarray(a)
    if dtype == "bf16":
        f = (arr.astype(np.uint32) << np.uint32(16)).view(np.float32)
    elif dtype == "f16":
        f = arr.astype(np.float16)
    else:
        f = arr.astype(np.float32)
    flat = [Fraction(float(v)) for v in f.reshape(-1)]
    return np.array(flat, dtype=object).reshape(arr.shape)


def e4m3_frac(byte: int):
    """E4M3 value as a Fraction by integer fields: sign, e = bits 6..3, m =
    bits 2..0; e == 0 -> m / 2^9; else (8 + m) * 2^(e - 10). None for NaN."""
    s = -1 if byte & 0x80 else 1
    e = (byte >> 3) & 0xF
    m = byte & 7
    if e == 15 and m == 7:
        return None
    if e == 0:
        return s * Fraction(m, 512)
    return s * Fraction(8 + m) * Fraction(2) ** (e - 10)


def e8m0_frac(byte: int):
    if byte == 255:
        return None
    return Fraction(2) ** (byte - 127)
