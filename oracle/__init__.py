"""CPU oracle for the quantized gated Delta-rule decode step.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product
library never does.  The arithmetic lives in ``stq_oracle.c`` (plain C,
binary64 update, binary32 encoding steps as defined); this module only
builds it and marshals numpy arrays.
"""
from .oracle import *  # noqa: F401,F403
