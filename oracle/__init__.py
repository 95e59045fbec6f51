"""fp64 CPU oracles of the fused chunked top-K KL loss and of the teacher top-K
cache writer -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does.
"""
from . import kl_oracle  # noqa: F401
from . import topk_oracle  # noqa: F401
from .kl_oracle import *  # noqa: F401,F403
