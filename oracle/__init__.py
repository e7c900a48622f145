"""CPU oracle (test infrastructure only).

Imported by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py``; never by the library or its binding. See ``qift_oracle.py``.
"""
from .qift_oracle import *  # noqa: F401,F403
from . import qift_oracle  # noqa: F401
