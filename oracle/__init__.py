"""fp64 CPU oracle for structured sparse causal attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP library and never calls it.

Every function here is written from the method pages' definitions (cited in
each docstring) in plain numpy fp64.  Pins that tie it to something other than
itself live in ``tests/test_oracle_pins.py``.  Parity status of each function:
all are pinned (see the pin list in that test module); none is "parity unpinned".
"""
from .sparse_attn_oracle import *  # noqa: F401,F403
