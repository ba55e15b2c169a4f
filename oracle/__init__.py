"""CPU oracle for the DBF linear forward -- test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package; the product path never does.
"""

from .dbf_oracle import *  # noqa: F401,F403
from .dbf_oracle import __all__  # noqa: F401
