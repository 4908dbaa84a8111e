"""Row-major GEMV, y[M] = A[M,N] . x[N], on MI355X (gfx950).

The compute lives in a hand-written HIP library behind a C ABI
(``include/gemv.h``); ``binding`` is a thin ctypes layer over it.  The
library is loaded on first use and its absence is an error: there is no CPU
fallback.
"""

from .binding import (  # noqa: F401,E402  (no library load at import time)
    GemvError,
    gemv_f32,
    gemv_f16,
    gemv_f16x32,
    gemv_f16_acc16,
    gemv_q8,
    gemv_q4,
    describe_launch,
    quantize_q8,
    quantize_q4,
    softmax_f16,
)
