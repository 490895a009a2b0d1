"""CPU oracle of the AWQ W4A16 path -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP product path never does.
"""
from .awq_oracle import *  # noqa: F401,F403
