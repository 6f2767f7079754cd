"""fp64 CPU oracle for grouped-query attention (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the product path never does.
"""
from .gqa_oracle import (attention_weights, band_visibility, expand_kv,
                         gather_paged, gqa, gqa_band, gqa_paged, group_size,
                         validate_shapes, visibility)

__all__ = ["attention_weights", "band_visibility", "expand_kv", "gather_paged", "gqa",
           "gqa_band", "gqa_paged", "group_size", "validate_shapes", "visibility"]
