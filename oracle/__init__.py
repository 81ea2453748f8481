"""Float64 CPU oracle for the chunked gated delta rule. TEST INFRASTRUCTURE ONLY.

Nothing in the library's product path may import, call, link or execute anything in this
package. Only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` use it. It shares no code with the HIP path.

* ``recurrence.gated_delta_rule``: the definition, a token-by-token float64 recurrence, as
  the kernel-test page (``r15_kernel_test.py``, function ``truth_f64``) and the model page
  (``model.py``, function ``delta_rule_reference``) state it.
* ``layer``: the layer steps on either side of the delta rule (gate prologue, causal depthwise
  conv + SiLU with tail continuation, gated RMSNorm), from the model page ``model.py``
  (functions ``_dn_gates``, ``_conv_silu``, ``_gated_rms``); pinned in
  ``tests/test_oracle_layer.py``.
* ``chunked.gated_delta_rule_chunked``: a second float64 formulation that evaluates the same
  recurrence C tokens at a time with an explicit matrix inverse. It exists only to pin the
  chunk algebra against the recurrence on tiny shapes.

Every function here is pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle.py``
(closed forms, invariants and brute-force comparisons); none is "parity unpinned".
"""
from .recurrence import gated_delta_rule, l2norm, guard
from .chunked import gated_delta_rule_chunked
from .layer import dn_gates, conv_silu, gated_rmsnorm

__all__ = ["gated_delta_rule", "gated_delta_rule_chunked", "l2norm", "guard", "dn_gates", "conv_silu",
           "gated_rmsnorm"]
