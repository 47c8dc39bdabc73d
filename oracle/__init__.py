"""CPU fp64 oracle (test infrastructure only; see egm_oracle's header)."""
from .egm_oracle import (  # noqa: F401
    BF16, EPILOGS, F16, GELU_C0, GELU_C1, TOLERANCE, add_bias, apply_epilog,
    gelu_tanh, product, reference, relu, relu_mask, round_to_bits, ulp, widen,
)
