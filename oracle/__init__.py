"""Plain, slow, CPU reference implementation of SegPagedAttention with head-aware KV reuse.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls, links or
runs this package: only the tests, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` do.  It shares no code with the HIP library or
its binding; the only thing both sides consume is the seeded input generator in
``synth``.

Everything is NumPy in fp64, written to be checked against the pages by eye:
  * ``oracle.tables``    - page allocation, per-head page tables, the visible
                           token set of each query, the relocation list.
  * ``oracle.rope``      - rotary position embedding and relocation of cached keys
                           as two literal rotations (back by the cached angle,
                           forward by the new one).
  * ``oracle.attention`` - softmax attention of each query over exactly its
                           visible tokens (gathered, no mask).
  * ``oracle.importance`` - the attention importance each context token
                           receives from the chunk's queries, and the top-k
                           token selection for the sparse FFN.
  * ``oracle.pack``      - per-head visible-page pack and unpack.

Every function is pinned by tests under ``tests/`` against closed forms, the
worked block-table example of the PagedAttention page, hand-written fixtures
and a brute-force dense masked attention; no function is "parity unpinned".
"""
from . import tables, rope, attention, importance, pack  # noqa: F401
