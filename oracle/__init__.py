"""CPU oracle for the 4-bit blockwise codec and its dequantize-and-multiply.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The product library never calls it and shares no code with it.
"""
from .qmv_oracle import *  # noqa: F401,F403
