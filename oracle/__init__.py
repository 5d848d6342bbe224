"""CPU fp64 oracle for the GEMM-epilogue hot path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package; the
product path (``transformer_gemm_epilogue_amd``) never does, and the two share no
code. See ``oracle/coda_oracle.py`` for the functions and the passages they follow.
"""
from .coda_oracle import *  # noqa: F401,F403
from .coda_oracle import __all__  # noqa: F401
