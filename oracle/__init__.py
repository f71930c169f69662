"""fp64 CPU oracle for exact attention forward/backward.

TEST INFRASTRUCTURE ONLY: imported by the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.
Every function carries "parity pinned" status in its own tests
(``tests/test_oracle.py``); none is unpinned.
"""

from .attention import *  # noqa: F401,F403
from .dropout import *  # noqa: F401,F403
from .attention import __all__ as _a
from .dropout import __all__ as _d

__all__ = list(_a) + list(_d)
