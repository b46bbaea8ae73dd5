"""fp64 CPU oracles (test infrastructure only; see trimul_ref, transition_ref and
attention_ref)."""
from .trimul_ref import (  # noqa: F401
    EPS, WEIGHT_FIELDS, line_operands, pair_update_ref, tri_mul_intermediates, tri_mul_ref,
    tri_mul_ref_lines, tri_mul_ref_pairs, tri_mul_residual_ref,
)
from .transition_ref import (  # noqa: F401
    TRANSITION_FIELDS, pair_transition_ref, pair_transition_update, transition_shapes,
)
from .attention_ref import (  # noqa: F401
    ATTENTION_FIELDS, NODES, attention_shapes, tri_attention_ref, tri_attention_ref_lines,
)
