"""fp64 CPU oracle of the cached flow-matching DiT step.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it. It shares no code with the HIP library; both are
written independently from the course pages on Qwen-Image-2.1 and are
compared element by element on the same seeded inputs.

Parity status of each function is listed in ``oracle/dit_oracle.py``.
"""
from .dit_oracle import *  # noqa: F401,F403
