"""CPU oracle for the forked KV cache -- TEST INFRASTRUCTURE, not part of the product.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The product path
(the HIP library and its Python binding) never does, and the two share no code:
the only module both sides use is ``workloads`` (seeded inputs and call
recipes), which contains none of the method's arithmetic.

What the oracle computes, and from which passage:

* ``allocator.FlatAllocator`` -- a deliberately naive block allocator in which
  every handle owns a flat list of (block id, valid count) entries and every
  block carries a sharer count and a sticky "frozen" bit.  Forking copies the
  parent's list (O(prefix) by design), which is the behaviour the library's
  O(1) tree must reproduce exactly.  It follows the copy-on-write description
  in the Dendrite article (ainews.cool, "technical deep dive": the shared prefix
  is stored once; forking at position t copies nothing below t and gives each
  branch new, empty leaves for positions >= t) and the "copy-on-write block
  table" named in the Dendrite demo tape ("the problem" section).
* ``cache.MaterializedCache`` -- keeps, for every handle, its own complete,
  contiguous token history; a fork duplicates it.  That is the full-copy
  strategy the article contrasts the method with (first option of its
  "technical deep dive"), used here only as the obviously correct reference.
* ``attention`` -- textbook softmax(q K^T / sqrt(d)) V in float64 over a
  materialised history, for decode (one query sees every token of its branch)
  and for verification of a block of draft tokens (query i sees positions up
  to its own), the parallel verification step of the DSpark blog (second layer).

Parity pins (closed forms, invariants, brute force and a library routine) live
in ``tests/test_oracle.py`` and ``tests/test_oracle_alloc.py``.  Readings where
the pages are silent are listed with each function.
"""
