"""CPU fp64 oracle for Newton–Schulz / Gram Newton–Schulz.

TEST INFRASTRUCTURE ONLY: imported by tests/, the package smoke check and the
bench's CPU-baseline leg, never by the product path.
"""
from .ns_oracle import (  # noqa: F401
    EPS,
    normalize,
    gram,
    quadratic,
    standard_ns,
    gram_ns,
    naive_gram_ns,
    ns_matrix,
    orthogonalize,
    composed_polynomial,
    theorem2_q,
    flops_standard,
    flops_standard_symmetric,
    flops_gram_naive,
    flops_gram_stable,
)
from .select_oracle import (  # noqa: F401
    n_selected,
    select_dim,
    l1_norms,
    select,
    select_orthogonalize,
)
