"""Float64 CPU oracle (test infrastructure only; see softmax_oracle)."""
from .softmax_oracle import cdf_ref, check_softmax_inputs, sample_ref, softmax_ref

__all__ = ["softmax_ref", "sample_ref", "cdf_ref", "check_softmax_inputs"]
