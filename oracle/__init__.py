"""Reference oracle for the deterministic attention backward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
C ABI or the Python binding in ``scheduling_persistent_attn_amd``) may import,
call, link or execute anything in this package.  Only ``tests/``, the smoke
check in ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.

The oracle is plain, slow and meant to be checked by eye against its sources:

* ``attention``  -- softmax attention forward/backward in float64 numpy, the
  textbook definition (the pages only require that the dQ reduction has a
  fixed order; the gradient itself is the standard one).
* ``schedule``   -- the four tile schedules (naive, descending-Q, shift,
  symmetric shift) written as explicit task lists and reduction ranks, from
  the DASH pages' prose (technical summary, section 2.2 A and B).
* ``dag``        -- the backward DAG of the DASH pages (technical summary,
  section 2.1), its critical path and the depth condition of their Lemma 1,
  in plain Python.

It shares no code with the HIP path.
"""
