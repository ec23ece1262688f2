"""fp64 CPU oracle for MLA prefill over a paged latent cache.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package. The HIP path never depends on it.
"""
from .mla_oracle import *  # noqa: F401,F403
