"""CPU oracle for the ClusterAttention forward path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg
may import this package. The HIP product path never does.
"""
from .clusterattn import *  # noqa: F401,F403
from . import clusterattn  # noqa: F401
