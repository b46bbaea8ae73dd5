"""fp64 CPU oracle (test infrastructure only; see trimul_ref)."""
from .trimul_ref import (  # noqa: F401
    EPS, WEIGHT_FIELDS, pair_update_ref, tri_mul_intermediates, tri_mul_ref, tri_mul_ref_pairs,
    tri_mul_residual_ref,
)
