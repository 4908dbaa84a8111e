"""CPU oracle for row-major GEMV, its weight quantiser and the row softmax
(test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding)
never imports, links or calls it, and it shares no code with them.
"""
from .oracle import (  # noqa: F401
    build,
    half_to_double,
    half_to_double_array,
    gemv_f32,
    gemv_f16,
    gemv_f16x32,
    gemv_q8,
    gemv_q4,
    num_threads,
    set_threads,
    library_path,
    double_to_half,
    quantize_q8,
    quantize_q4,
    quant_rmse,
    softmax_f16,
)
from .metrics import (  # noqa: F401
    parity_error,
    parity_report,
    GATES,
    acc16_bound,
    acc16_ratio,
    softmax_error,
    SOFTMAX_GATE,
)
