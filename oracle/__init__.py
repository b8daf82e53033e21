"""CPU oracle for the MoVA routed value projection.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or calls
this package; only the tests, the smoke check and the benchmark's CPU
baseline leg do.  It is a plain, slow, obviously correct float64
implementation written from the pages describing the method, and it shares
no code with the HIP path.

Parity status per function (details in the module docstring of
``oracle.mova_oracle``):

* ``router_logits``, ``sigmoid``, ``route`` (except the bias role and the
  router's reduction order), ``combine_experts``, ``value_forward`` and
  ``dense_value_proj`` (the matched dense baseline) and
  ``paged_value_write`` (the paged cache store), ``rebuild_values`` (the
  compact cache's reconstruction), ``pack_routing_record`` /
  ``unpack_routing_record`` / ``rebuild_from_record`` (the compact cache's
  record), ``swiglu_expert`` and ``ffn_moe_forward``
  (the FFN mixture of experts): pinned by the tests in
  ``tests/test_oracle_pins.py``;
* the role of the router bias (added to the scores for selection only) and
  the router's summation order: parity unpinned -- no page prints a value
  that fixes them; they are documented readings.
"""
from .mova_oracle import (  # noqa: F401
    BIAS_ROLES,
    Routing,
    combine_experts,
    dense_value_proj,
    ffn_moe_forward,
    swiglu_expert,
    paged_value_write,
    pack_routing_record,
    rebuild_from_record,
    rebuild_values,
    unpack_routing_record,
    route,
    router_logits,
    sigmoid,
    silu,
    value_forward,
)
