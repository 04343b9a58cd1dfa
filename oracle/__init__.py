"""CPU oracle for the pooled-embedding path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package. The HIP library never calls it and shares no code with it.
"""
from .embedding_oracle import *  # noqa: F401,F403
