"""CPU oracle for the delta-rule memory operator -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its binding) never
imports, calls or links anything here, and this package imports nothing from
the product path.

Contents:
  recurrence.forward / recurrence.backward -- the token-by-token float64
  recurrence of the pages' update rule, and its manual reverse mode;
  recurrence.gates_from_logits / logit_gradients -- the gate activations of the workloads
  (sigmoid, exp(-softplus)) and their chain rule, for gates given as logits.
"""
from .recurrence import backward, forward, gates_from_logits, logit_gradients  # noqa: F401
