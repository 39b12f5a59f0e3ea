"""fp64 CPU oracle (test infrastructure only; never imported by the library)."""
from .attention import (CAP_METHODS, Params, backward, cap_derivative, cap_forward,
                        dkv_keys, dq_rows, forward, preprocess, ranker_bounds_from_segments,
                        sigmoid, unmasked_pairs, visible)

__all__ = ["CAP_METHODS", "Params", "backward", "cap_derivative", "cap_forward", "dkv_keys",
           "dq_rows", "forward", "preprocess", "ranker_bounds_from_segments", "sigmoid",
           "unmasked_pairs", "visible"]
