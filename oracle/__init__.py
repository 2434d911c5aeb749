"""Float64 CPU oracle for row-wise softmax cross-entropy (TEST INFRASTRUCTURE).

This package is the checker, not the product.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The HIP library never calls it, and it never calls the HIP
library: the two share no code, and only the seeded input generators in
``softmax_cross_entropy_amd/inputs.py`` feed both.

It writes out the plain definitions in float64 NumPy:

* ``oracle.ce``: the per-row loss, the log-sum-exp and the gradient of
  softmax cross-entropy.
* ``oracle.lce``: the linear cross-entropy forward and its gradients dH, dW.  It
  materialises the logits H.W^T in float64 row blocks and applies ``oracle.ce``.
* ``oracle.ce_options``: label smoothing, probability targets, ignore_index and
  the sum / mean reductions of the cross-entropy, with their gradients.
* ``oracle.kl``: the row-wise KL divergence of a teacher row from a student row
  and its gradient with respect to the student logits.
* ``oracle.js``: the row-wise Jensen-Shannon divergence of the two rows and its
  gradient with respect to the student logits.

Every function is pinned by ``tests/test_oracle*.py`` against values the pages
print, closed forms, invariants and brute force.  No function here is
"parity unpinned".
"""

from . import ce, ce_options, js, kl, lce  # noqa: F401
