"""Float64 CPU oracle for 1.5-entmax attention and row-wise alpha-entmax.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, helpers, tables or pre/post-processing), and it
imports nothing from ``entmax_amd``.

Sources (the pages this follows, cited by title and section):

* "ADASPLASH -- ROBERTA Benchmark Result" (AdaSplash Attention module
  specification): section 2.1 (Tsallis entropy, variational definition),
  section 2.2 Theorem 1 (closed form p = [(s - tau)/2]_+^2 with sum p = 1),
  section 2.3 Theorem 2 (monotone g, bisection), section 2.4 (Jacobian),
  section 3 (masking order: padding, causal, splash window).
* "RoBERTa Base with AdaSplash Attention" model card: Architecture Overview
  (S = Q K^T / 8, O_i = sum_{A_ij > 0} A_ij V_j), Mathematical Formulation 1-2.
* "DistilBERT SST-2 with AdaSplash Attention" model card: Mathematical
  Formulation 2 (bracket [max - 2, max - 2/sqrt(L)]) and 3 (exact zeros).
* "ADASPLASH -- ROBERTA Benchmark Result", section 4 (the entmax_bisect
  routine for any alpha in (1, 2]): ``entmax_alpha.py``.

Every function is pinned by CPU tests in ``tests/test_oracle*.py`` against
closed forms (the 1.5 closed form, sparsemax at alpha = 2), brute-force
support enumeration, an independent bisection, the softmax limit as alpha
goes to 1, the variational objective and finite differences.  No function here is
"parity unpinned".
"""

from .entmax15 import (  # noqa: F401
    allowed_mask,
    entmax15_backward,
    entmax15_exact,
    entmax15_bisect,
    attention_forward,
    attention_backward,
    attention_decode,
    attention_decode_backward,
    tsallis15_objective,
)
from .entmax_alpha import (  # noqa: F401
    entmax_alpha_backward,
    entmax_alpha_vjp,
    entmax_alpha_bisect,
    entmax_alpha_exact,
    tsallis_objective,
)
