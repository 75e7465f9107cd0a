"""CPU oracle for the Qwen3.5 hybrid decode path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``, never by the product path.

Parity pinned: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, special cases, library routines or brute force.  The
layer and stack compositions are pinned only through their parts (the pages
print no worked example): "parity unpinned" beyond composition.
"""
from .qwen35 import *  # noqa: F401,F403
from . import qwen35  # noqa: F401
from . import turbo8  # noqa: F401
from . import turbo_lm  # noqa: F401
from . import prefill  # noqa: F401
