"""Plain, slow fp64 CPU oracle for StreamKL.  TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the `cpu_baseline` leg of `bench.py` may import
this package. The product path (the HIP library and its Python binding) never imports, calls
or links anything here, and this package imports nothing from the product path.

It computes the per-query-row KL divergence KL(P1 || P2) between two attention distributions
P_t = softmax(scale * Q_t K_t^T) and the gradients of the two backward settings, by the plain
definition, materialising the logits of one block of query rows at a time in float64.
See `oracle.reference` for the functions and the passages each follows.
"""
from .reference import (  # noqa: F401
    logits_block, forward_slice, backward_slice, dk_rows_slice, forward, backward,
)
