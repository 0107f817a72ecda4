"""CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  The GPU
library never imports it and it never imports the GPU library.
"""
from . import attention, radix_ref  # noqa: F401
