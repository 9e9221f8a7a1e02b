"""MI355X (gfx950) SMOE routed-expert MoE FFN: HIP kernels behind a C ABI.

The compute lives in ``libsmoe.so`` (sources in ``csrc/``, ABI in
``include/smoe.h``); :mod:`.binding` is a ctypes binding with the same
function names. Build with ``__graft_entry__.build()``.
"""

from .binding import *  # noqa: F401,F403
from .binding import EXPORTED, LIB_PATH, SmoeError, load_library  # noqa: F401
from .vault import *  # noqa: F401,F403
from .offload import *  # noqa: F401,F403
