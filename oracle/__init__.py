"""CPU oracle for the SMOE routed-expert FFN (test infrastructure only).

Only the test suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product
library never imports, links or calls it.
"""

from .smoe_oracle import *  # noqa: F401,F403
from . import smoe_vault  # noqa: F401
