"""CPU oracle for the decode-step linear layer (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this
package imports nothing from it.

``oracle.c`` holds the arithmetic (fp64, sequential k); this module only
builds it with gcc, loads it with ctypes and marshals numpy arrays.
"""
from .oracle import (  # noqa: F401
    LIB_PATH,
    bf16_from_f64,
    bf16_value,
    build,
    dequant_i8,
    dequant_q4g64,
    f16_from_f64,
    f16_value,
    gemm_dense,
    gemm_f64w,
    gemm_i8,
    gemm_q4g64,
    load,
    open_lib,
    quantize_i8,
    quantize_q4g64,
    residual_add,
    rmsnorm,
    swiglu,
    use,
)
