"""Algorithmic byte and FLOP counts, and the rate arithmetic built on them.

Byte model ("Making GEMV Fast", section "Arithmetic intensity", table
"Memory Access"): every element of A is read once, x is read once (kept in
cache), y is written once.  For FP32 that totals 4(MN + N + M) bytes.  The
same rule applied to the other storage formats, counting the binary16 scales
of the quantised formats as bytes that must be streamed ("membound", section
"The kernel decode actually runs: dequant GEMV", where the INT4 group scales
add 2/128 byte per weight):

    f32 : 4MN            + 4N + 4M
    f16 : 2MN            + 2N + 4M
    f16x32 : 2MN         + 4N + 4M      (FP16 weights, FP32 activations)
    f16_acc16 : as f16                  (FP16 accumulation changes no byte)
    q8  :  MN + 2M       + 2N + 4M      (one binary16 scale per row)
    q4  : MN/2 + 2M(N/128) + 2N + 4M    (one binary16 scale per 128-column group)

FLOP model ("Making GEMV Fast", section "Computation"): N multiplications and
N - 1 additions per row, M(2N - 1) = 2MN - M in total.  Dequantisation
multiplies are not counted as FLOPs.
"""
from __future__ import annotations

X_BYTES = {"f32": 4, "f16": 2, "f16x32": 4, "f16_acc16": 2, "q8": 2, "q4": 2}


def weight_bytes(kind: str, M: int, N: int) -> int:
    """Bytes of A plus its scales: the streamed, read-once part."""
    if kind == "f32":
        return 4 * M * N
    if kind in ("f16", "f16x32", "f16_acc16"):
        return 2 * M * N
    if kind == "q8":
        return M * N + 2 * M
    if kind == "q4":
        if N % 128:
            raise ValueError("INT4 needs N % 128 == 0")
        return (M * N) // 2 + 2 * M * (N // 128)
    raise ValueError(kind)


def alg_bytes(kind: str, M: int, N: int) -> int:
    return weight_bytes(kind, M, N) + X_BYTES[kind] * N + 4 * M


def flops(M: int, N: int) -> int:
    return 2 * M * N - M if N > 0 else 0


def gbps(nbytes: float, seconds: float) -> float:
    return nbytes / seconds / 1e9


def arithmetic_intensity(kind: str, M: int, N: int) -> float:
    return flops(M, N) / alg_bytes(kind, M, N)


def ratio(t_ref: float, t_other: float) -> float:
    """Speedup of ``other`` over ``ref`` from their times (x-fp16 column)."""
    return t_ref / t_other


def quant_bytes(kind: str, M: int, N: int) -> int:
    """Algorithmic bytes of one quantiser call: FP32 weights read once; codes,
    binary16 scales and the per-row squared error (FP32) written once."""
    if kind == "q8":
        return 4 * M * N + M * N + 2 * M + 4 * M
    if kind == "q4":
        return 4 * M * N + M * N // 2 + 2 * M * (N // 128) + 4 * M
    raise ValueError(kind)


def softmax_bytes(M: int, N: int) -> int:
    """One read and one write of every binary16 element ("membound", online
    softmax section: a balanced stream)."""
    return 4 * M * N


def ring_copies(kind: str, M: int, N: int, min_bytes: int = 1 << 30) -> int:
    """Weight copies needed so that a rotation streams >= min_bytes."""
    wb = weight_bytes(kind, M, N)
    return max(1, -(-min_bytes // wb))
