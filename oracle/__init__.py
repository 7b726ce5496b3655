"""Float64 CPU oracle (test infrastructure only; see softmax_oracle)."""
from .softmax_oracle import (allowed_bits_to_bool, cdf_ref, check_softmax_inputs, sample_ref,
                             softmax_masked_ref, softmax_ref)

__all__ = ["softmax_ref", "sample_ref", "cdf_ref", "check_softmax_inputs", "allowed_bits_to_bool",
           "softmax_masked_ref"]
