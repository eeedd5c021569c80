"""CPU oracle for the MoE expert layer.  TEST INFRASTRUCTURE, not product code.

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The HIP library and
its Python binding never do, and this package imports nothing from them.
"""
from . import moe_oracle, brute  # noqa: F401
