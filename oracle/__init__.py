"""fp64 CPU oracle for hybrid-head prefill attention (Elastic Attention).

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
reference that the HIP path is checked against.  Only the test suite, the
package smoke check and the benchmark's CPU-baseline leg may import or run it;
the product path never does.  It shares no code with the HIP library: it reads
the same bf16 inputs (widened exactly to float64) and computes everything in
float64 with numpy.

Modules
  attention  masked softmax attention for FA / SSA / XA heads (Eqs. 1-3)
  xa         antidiagonal block scoring and the top-mass block selector
  ratios     Omega_MSR / Omega_ESR and the per-head pruning rate rho (Eqs. 4-5)
  router     the Attention Router's inference pass: boundary pooling of the
             key states, Task MLP, Router MLP, arg max
  decode     one decode step: the newest token of each sequence over the
             keys its head's mode keeps

Parity status of each function is stated in its module header.
"""

from . import attention, xa, ratios, router, decode  # noqa: F401
