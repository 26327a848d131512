"""CPU oracle for rollout-guided FP4 fake-quant (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does.  The arithmetic lives in ``trace_oracle.c``;
this module only compiles and loads it and marshals numpy arrays.
"""
from .oracle import *  # noqa: F401,F403
