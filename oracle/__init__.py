"""CPU oracle for paged decode attention.  TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation of what the paged decode
path computes, written from the PagedAttention explainer pages and used only
by the tests, the smoke check and the CPU-baseline leg of the benchmark.  The
product path never imports, calls or links anything here, and nothing here
imports the product path.

Modules
-------
attention      scaled dot-product decode attention over a contiguous context,
               and the log-sum-exp merge of partial softmax states (fp64).
cache          the slot-mapped cache write, the block copy and the gather of a
               sequence through its block table, on a logical pool
               ``[num_blocks, num_kv_heads, block_size, head_dim]``.
layout         the documented physical block layout of the HIP library's K and
               V pools, as a view onto the logical pool (an encoding).
block_manager  a pure-Python block manager: LIFO free list, reference counts,
               fork and copy-on-write.

Pins: every function is checked in ``tests/test_oracle_*.py`` against values
the pages print (``tests/golden/``), closed forms, invariants and brute force
on tiny inputs.  No function here is "parity unpinned".
"""

from . import attention, block_manager, cache, layout  # noqa: F401
