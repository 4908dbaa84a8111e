"""Test-side construction of quantised operands from chosen integer values.

The INT4 storage rule (two signed nibbles per byte, the low nibble holding
the even column, two's complement) is written out here independently of both
the oracle's decoder and the HIP kernels, so that a test can choose q values
and know exactly what each column must contribute.
"""
import numpy as np


def pack_int4(q: np.ndarray) -> np.ndarray:
    """q: integer [M, N] with values in [-8, 7], N even -> uint8 [M, N/2]."""
    q = np.asarray(q, dtype=np.int64)
    if q.min(initial=0) < -8 or q.max(initial=0) > 7:
        raise ValueError("INT4 values must lie in [-8, 7]")
    codes = (q & 0xF).astype(np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Vectorised inverse of pack_int4 (independent of the C oracle)."""
    p = np.asarray(packed, dtype=np.uint8)
    M, half = p.shape
    codes = np.empty((M, 2 * half), dtype=np.int64)
    codes[:, 0::2] = p & 0xF
    codes[:, 1::2] = p >> 4
    return np.where(codes >= 8, codes - 16, codes)


def f16(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float16)
