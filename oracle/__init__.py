"""CPU oracle for the Moshi RQ-Transformer frame step.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import or run anything in this package.  The product path (the HIP
library and its Python binding) never calls it, and shares no code with it.
"""
from .moshi_oracle import *  # noqa: F401,F403
