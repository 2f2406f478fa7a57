"""CPU fp64 oracle for block-causal attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never calls it and shares no code with it.

The arithmetic lives in ``attn_oracle.c`` (plain C, double precision, OpenMP
over independent problems), compiled with gcc by ``build()``.  This module is
argument marshalling only: it widens the inputs to float64, calls the C entry
points, and returns float64 numpy arrays.

Parity status: every function here is pinned by ``tests/test_oracle.py``
(torch CPU fp64 SDPA with an explicit boolean mask and autograd, closed forms,
backward identities, finite differences, invariants, and planted-mistake
checks); none is "parity unpinned".
"""
from .oracle import (build, lib_path, set_threads, max_threads, space_fwd, space_bwd,
                     time_fwd, time_bwd, fwd, bwd)

__all__ = ["build", "lib_path", "set_threads", "max_threads", "space_fwd", "space_bwd",
           "time_fwd", "time_bwd", "fwd", "bwd"]
