"""CPU oracle (fp64) for the tensor-parallel linear pair.

Test infrastructure only: tests/, ``__graft_entry__.smoke()`` and bench.py's
``cpu_baseline`` leg may use it; the product path never does.
"""
from .tp_oracle import *  # noqa: F401,F403
from .tp_oracle import __all__  # noqa: F401
