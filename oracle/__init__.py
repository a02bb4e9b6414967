"""CPU oracle of the routed MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library under
``mixture_experts_routed_lineargate_amd``) never imports or calls it.
"""
from . import moe_oracle, scalar  # noqa: F401
