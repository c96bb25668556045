"""CPU oracle for paged attention -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  It shares no code with the HIP
library in ``paged_kv_cache_87_amd``.
"""

from .paged_attention import *  # noqa: F401,F403
from .paged_attention import __all__  # noqa: F401
