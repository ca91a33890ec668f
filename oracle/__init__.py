"""CPU oracle of the routed-MoE verify layer -- test infrastructure only.

Importable only from ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product path (the HIP library and
its Python binding) never imports it.
"""

from . import moe_oracle, scalar_twin  # noqa: F401
