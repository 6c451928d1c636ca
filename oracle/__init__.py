"""CPU oracle for the hybrid-batch paged-attention step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct restatement of what the step computes, used
to check the HIP path.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the
product library (``chunked_prefill_decode_amd``) and imports nothing from it.

Modules
  * ``attention`` -- fp64 causal softmax attention over contiguous per-request
    K/V (what a decode row and a prefill-chunk row compute).
  * ``scheduler`` -- the stall-free batch builder (decodes first, then
    unfinished prefill chunks, then admissions under the token budget) with a
    FIFO page pool and a request state machine.
  * ``kvcache``   -- what a paged KV append must leave in the cache.
  * ``linear``    -- fp64 token-batch linear layer y = x w^T (the GEMMs on
    either side of attention).

Every function is pinned by ``tests/test_oracle_*.py`` against facts the pages
and the mathematics fix (closed forms, invariants, library special cases,
brute force).  No function here is "parity unpinned".
"""
