"""CPU oracle for iS-KV's online low-rank KV compression (test infrastructure).

This package is test infrastructure only. It may be imported, called or run
by ``tests/``, by ``__graft_entry__.smoke()`` and by ``bench.py``'s
``cpu_baseline`` leg, and by nothing else: the product path never routes
through it, and it shares no code with the HIP library.

It is a plain, slow, deliberately literal NumPy/LAPACK implementation of what
the pages describe, in float64 by default (float32 on request), following the
U / Sigma / B notation of the pages rather than the GPU path's storage choices.
Every function cites the passage it follows: the page is Zhongzhu Zhou's
reading notes on "iS-KV: Online Low-Rank KV Cache Compression via
Block-Incremental SVD" (cited as "iS-KV notes"), with its section, equation,
algorithm or table.

Parity status: every function is pinned by a closed form, an invariant, a
worked example from the pages or brute force in ``tests/test_oracle_*.py``,
except the whole-stream runs over thousands of rows, whose only check beyond
those pins is the float64-versus-float32 cross-check (parity unpinned beyond
the per-merge pins).
"""
from .iskv_oracle import *  # noqa: F401,F403
from .iskv_oracle import __all__  # noqa: F401
