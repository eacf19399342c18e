"""CPU oracle of the integer-only attention core.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline import this package; the product path never does.
"""
from .oracle import (  # noqa: F401
    build, forward, softmax_row, requant, requant_array, shift_exp, ilog2r,
    check_params, library_path, linear, shiftgelu, isqrt10, ilayernorm, linattn,
)
