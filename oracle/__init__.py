"""fp64 CPU oracle for one context-parallel rank's share of causal THD attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import or
run anything in this package. It shares no code, constants or helpers with the
HIP library, and the library never calls it.

See ``oracle/thd.py`` for the definitions and the pages each one follows.
"""
from .thd import *  # noqa: F401,F403
