"""CPU oracle for the W4A16 quantized linear layer.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product path never does.
It shares no code with the HIP library.

The arithmetic lives in ``w4a16_oracle.c`` (plain C, built with gcc); this
package holds the ctypes marshalling and the build step.
"""
from .oracle import (  # noqa: F401
    ACT_GELU_TANH,
    ACT_SWIGLU,
    BF16,
    F16,
    F32,
    GROUP,
    act_value,
    activate,
    bf16_to_double,
    build,
    codes_to_nibbles,
    dequantize,
    f16_to_double,
    library_path,
    linear,
    linear_act,
    linear_entries,
    nibbles_to_codes,
    num_threads,
    quantize,
    quantize_int8,
    round16,
    splitmix64,
    uniform,
    update,
)
