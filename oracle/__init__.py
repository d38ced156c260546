"""Test infrastructure only: the fp64 CPU oracle for the transposed convolution
and its epilogues.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package; the library path never
does."""
from .oracle import *  # noqa: F401,F403
