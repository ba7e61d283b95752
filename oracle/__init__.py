"""CPU oracle (test infrastructure only; see ``tq_oracle``).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  The product library never does.
"""
from .tq_oracle import *  # noqa: F401,F403
