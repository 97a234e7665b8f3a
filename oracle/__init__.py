"""CPU oracle for one tensor-parallel rank's share of a DiT block.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The HIP library never calls it, and
it shares no code with the HIP path.

It is plain numpy in float64 (BLAS matmuls accumulate in float64), written from
the Diffusers tensor-parallelism pages ("Paralelismo de tensor", and its
v0.43.0 Chinese twin "张量并行") and the context-parallelism page
("Paralelismo de contexto"): each function cites the section it follows.
Every function is pinned by CPU tests against closed forms, brute force,
library routines or the pages' invariants; none is "parity unpinned".
"""
from .tp_block import *  # noqa: F401,F403
from .cp_attention import *  # noqa: F401,F403
